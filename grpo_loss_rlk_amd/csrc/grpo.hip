// GRPO / DAPO token loss over a packed ragged batch of responses.
//
// LumenRL README, "Key Features" (GRPO, DAPO, PPO) and "Rollout Correction"
// (TIS: large importance ratios are clipped); RL-Kernel ROCm sparse performance
// page: KL coefficient 0.01 (quick-start command), GRPO standard-deviation
// normalisation with eight samples per prompt (profile paragraph).
//
//   A_j   = (r_j - mean_g r) / (std_g r + eps)        groups of `group_size`
//   rho   = exp(lp_new - lp_old),  rho~ = min(rho, C)
//   s     = min(rho~ A, clip(rho~, 1 - eps_low, 1 + eps_high) A)
//   k3    = exp(lp_ref - lp_new) - (lp_ref - lp_new) - 1
//   l_t   = -s + beta k3,   loss = sum_t l_t / T_tot
//   dL/dlp_new = (-A rho [live branch] + beta (1 - exp(lp_ref - lp_new))) / T_tot
//
// Variants (prime-rl v0.10.0 release notes, "2. RL Algorithms" and "Breaking
// changes"; LumenRL README, "Rollout Correction"): IPO / IcePop masks, the
// CISPO constant clipped weight, MIS ratio normalisation, a length-weighted
// baseline, zero-advantage filtering and prompt-mean aggregation; the token
// weights replace 1 / T_tot.
//
// Launches: advantages (one thread per group), token weights and the check of
// cu_seqlens (one block, fixed order), for MIS the ratio mean (fixed
// 256-token blocks, then one block), per-token terms (one thread per token,
// fixed 256-token blocks, per-block fp64 partial sums), and a single-block
// fixed-order fold. Every split depends only on the sizes, so the loss is
// bitwise reproducible. cu_seqlens is read in device memory only (no host
// copy), so a call can be captured in a graph; offsets that are not
// non-decreasing from 0 to n_tokens make every float output NaN and set the
// status word.
#include "common.h"
#include "kernels.h"

namespace rlk {

namespace {

constexpr int kTB = 256;
constexpr int kNMetric = 5;   // sum l, clip count, TIS count, sum k3, sum rho

struct Ws {
  const int64_t* cu;   // the caller's device offsets
  double* adv;
  double* resp_w;    // [n_seqs] token weight of each response
  double* scal;      // [0] MIS ratio mean, [1] tokens entering the loss,
                     // [2] 1 when cu_seqlens is valid, else 0
  double* rho_part;  // [n_blocks] MIS partial sums
  double* partial;   // [n_blocks][kNMetric]
};

size_t slot(size_t bytes) { return (bytes + 255) / 256 * 256; }

Ws carve(void* workspace, const int64_t* cu, int64_t n_tokens, int64_t n_seqs) {
  char* p = reinterpret_cast<char*>(workspace);
  const size_t nb = size_t((n_tokens + kTB - 1) / kTB);
  Ws w;
  w.cu = cu;
  w.adv = reinterpret_cast<double*>(p);
  p += slot(size_t(n_seqs) * 8);
  w.resp_w = reinterpret_cast<double*>(p);
  p += slot(size_t(n_seqs) * 8);
  w.scal = reinterpret_cast<double*>(p);
  p += slot(4 * 8);
  w.rho_part = reinterpret_cast<double*>(p);
  p += slot(nb * 8);
  w.partial = reinterpret_cast<double*>(p);
  return w;
}

__global__ __launch_bounds__(kTB) void grpo_advantages(GrpoArgs a, Ws w) {
  const int64_t g = int64_t(blockIdx.x) * kTB + threadIdx.x;
  if (a.advantages) {
    if (g < a.n_seqs) w.adv[g] = double(a.advantages[g]);
    return;
  }
  const int G = a.group_size;
  if (g >= a.n_seqs / G) return;
  const float* r = a.rewards + g * G;
  // a group whose rewards are all equal carries no signal: A = 0 exactly
  // (also with adv_eps = 0, where the quotient below would be 0/0)
  bool constant = true;
  for (int j = 1; j < G; ++j) constant = constant && r[j] == r[0];
  if (constant) {
    for (int j = 0; j < G; ++j) w.adv[g * G + j] = 0.0;
    return;
  }
  double mu = 0.0;
  for (int j = 0; j < G; ++j) mu += double(r[j]);
  mu /= double(G);
  double b = mu;
  if (a.baseline == 1) {   // length-weighted: sum_j L_j r_j / sum_j L_j
    double lr = 0.0, ls = 0.0;
    for (int j = 0; j < G; ++j) {
      const double L = double(w.cu[g * G + j + 1] - w.cu[g * G + j]);
      lr += L * double(r[j]);
      ls += L;
    }
    if (ls > 0.0) b = lr / ls;
  }
  double ss = 0.0;
  for (int j = 0; j < G; ++j) {
    const double d = double(r[j]) - mu;
    ss += d * d;
  }
  const double sd = sqrt(ss / double(G - a.std_ddof));
  for (int j = 0; j < G; ++j) {
    double A = double(r[j]) - b;
    if (a.normalize_std) A /= (sd + double(a.adv_eps));
    w.adv[g * G + j] = A;
  }
}

// Token weight of each response (one block, fixed order): token mean 1 /
// T_kept; prompt mean 1 / (G_kept T_g); 0 for a filtered response. The same
// block checks cu_seqlens (cu[0] = 0, non-decreasing, cu[n_seqs] = n_tokens)
// and writes the advantages out (NaN when the offsets are invalid).
__global__ __launch_bounds__(kTB) void grpo_weights(GrpoArgs a, Ws w) {
  __shared__ double sd[kTB / kWave];
  const int tid = threadIdx.x;
  double bad = 0.0;
  for (int64_t j = tid; j < a.n_seqs; j += kTB) bad += w.cu[j + 1] < w.cu[j] ? 1.0 : 0.0;
  if (tid == 0) bad += (w.cu[0] != 0 || w.cu[a.n_seqs] != a.n_tokens) ? 1.0 : 0.0;
  const bool valid = block_sum(bad, sd) == 0.0;
  if (a.adv_out)
    for (int64_t j = tid; j < a.n_seqs; j += kTB)
      a.adv_out[j] = valid ? float(w.adv[j]) : __builtin_nanf("");
  if (tid == 0) w.scal[2] = valid ? 1.0 : 0.0;
  auto kept = [&](int64_t j) { return !(a.filter_zero_adv && w.adv[j] == 0.0); };
  auto len = [&](int64_t j) { return double(w.cu[j + 1] - w.cu[j]); };
  if (a.aggregation == 0) {
    double t = 0.0;
    for (int64_t j = tid; j < a.n_seqs; j += kTB) t += kept(j) ? len(j) : 0.0;
    const double T_kept = block_sum(t, sd);
    const double inv = T_kept > 0.0 ? 1.0 / T_kept : 0.0;
    for (int64_t j = tid; j < a.n_seqs; j += kTB) w.resp_w[j] = kept(j) ? inv : 0.0;
    if (tid == 0) w.scal[1] = T_kept;
    return;
  }
  const int G = a.group_size;
  const int64_t n_groups = a.n_seqs / G;
  auto group_tokens = [&](int64_t g) {
    double tg = 0.0;
    for (int j = 0; j < G; ++j) tg += kept(g * G + j) ? len(g * G + j) : 0.0;
    return tg;
  };
  double cnt = 0.0, tot = 0.0;
  for (int64_t g = tid; g < n_groups; g += kTB) {
    const double tg = group_tokens(g);
    cnt += tg > 0.0 ? 1.0 : 0.0;
    tot += tg;
  }
  const double G_kept = block_sum(cnt, sd);
  const double T_kept = block_sum(tot, sd);
  for (int64_t g = tid; g < n_groups; g += kTB) {
    const double tg = group_tokens(g);
    const double inv = (G_kept > 0.0 && tg > 0.0) ? 1.0 / (G_kept * tg) : 0.0;
    for (int j = 0; j < G; ++j) w.resp_w[g * G + j] = kept(g * G + j) ? inv : 0.0;
  }
  if (tid == 0) w.scal[1] = T_kept;
}

// response owning token t: last j with cu[j] <= t (cu is non-decreasing)
RLK_DEV int64_t owner(const Ws& w, int64_t n_seqs, int64_t t) {
  int64_t lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (w.cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// MIS: per-block sums of the ratio over tokens entering the loss, then the mean
__global__ __launch_bounds__(kTB) void grpo_rho_part(GrpoArgs a, Ws w) {
  __shared__ double sd[kTB / kWave];
  const int64_t t = int64_t(blockIdx.x) * kTB + threadIdx.x;
  double v = 0.0;
  if (t < a.n_tokens && w.resp_w[owner(w, a.n_seqs, t)] > 0.0)
    v = exp(double(a.lp_new[t]) - double(a.lp_old[t]));
  v = block_sum(v, sd);
  if (threadIdx.x == 0) w.rho_part[blockIdx.x] = v;
}

__global__ __launch_bounds__(kTB) void grpo_rho_fold(Ws w, int64_t n_blocks) {
  __shared__ double sd[kTB / kWave];
  double v = 0.0;
  for (int64_t b = threadIdx.x; b < n_blocks; b += kTB) v += w.rho_part[b];
  v = block_sum(v, sd);
  if (threadIdx.x == 0) w.scal[0] = w.scal[1] > 0.0 ? v / w.scal[1] : 1.0;
}

__global__ __launch_bounds__(kTB) void grpo_tokens(GrpoArgs a, Ws w) {
  __shared__ double sd[kTB / kWave];
  const int64_t t = int64_t(blockIdx.x) * kTB + threadIdx.x;
  double acc[kNMetric] = {0, 0, 0, 0, 0};
  if (t < a.n_tokens && w.scal[2] == 0.0) {   // invalid offsets: NaN outputs
    const float nan = __builtin_nanf("");
    a.grad[t] = nan;
    if (a.token_loss) a.token_loss[t] = nan;
    if (a.token_flags) a.token_flags[t] = 0;
  } else if (t < a.n_tokens) {
    const int64_t j = owner(w, a.n_seqs, t);
    const double A = w.adv[j], wt = w.resp_w[j];
    const double C = a.tis_cap, lo_b = 1.0 - double(a.eps_low), hi_b = 1.0 + double(a.eps_high);
    const double beta = a.kl_coef;
    const double lpn = a.lp_new[t], lpo = a.lp_old[t];
    const double rho = exp(lpn - lpo);
    double rt;
    bool tis, ratio_live;
    if (a.correction == 1) {   // MIS
      rt = rho / w.scal[0];
      tis = false;
      ratio_live = true;
    } else {                   // TIS
      rt = rho < C ? rho : C;
      tis = rho > C;
      ratio_live = rho <= C;
    }
    double s, g_ratio;
    bool flag2;
    if (a.loss_type == 0) {          // DAPO clipped surrogate
      const double clipped = rt < lo_b ? lo_b : (rt > hi_b ? hi_b : rt);
      const double s1 = rt * A, s2 = clipped * A;
      s = s1 < s2 ? s1 : s2;
      flag2 = (A > 0.0 && rt > hi_b) || (A < 0.0 && rt < lo_b);
      g_ratio = (ratio_live && !flag2) ? -A * rt : 0.0;
    } else if (a.loss_type == 4) {   // detached TIS weight on an on-policy surrogate
      s = rt * A;
      flag2 = false;
      g_ratio = -A * rt;
    } else if (a.loss_type == 3) {   // CISPO: constant clipped weight on lp_new
      const double wc = rt < lo_b ? lo_b : (rt > hi_b ? hi_b : rt);
      s = wc * A * lpn;
      flag2 = rt < lo_b || rt > hi_b;
      g_ratio = -A * wc;
    } else {                         // IPO / IcePop masks
      const bool m = a.loss_type == 1
                         ? fabs(exp(lpn) - exp(lpo)) <= double(a.ipo_eps)
                         : (rho >= double(a.icepop_lo) && rho <= double(a.icepop_hi));
      s = m ? rt * A : 0.0;
      flag2 = !m;
      g_ratio = (m && ratio_live) ? -A * rt : 0.0;
    }
    double k3 = 0.0, ed = 1.0;
    if (a.lp_ref) {
      const double delta = double(a.lp_ref[t]) - lpn;
      ed = exp(delta);
      k3 = ed - delta - 1.0;
    }
    const double ell = -s + beta * k3;
    a.grad[t] = float(wt * (g_ratio + beta * (1.0 - ed)));
    if (a.token_loss) a.token_loss[t] = float(ell);
    if (a.token_flags) a.token_flags[t] = uint8_t((tis ? 1 : 0) | (flag2 ? 2 : 0));
    acc[0] = wt * ell;
    acc[1] = flag2 ? 1.0 : 0.0;
    acc[2] = tis ? 1.0 : 0.0;
    acc[3] = k3;
    acc[4] = rho;
  }
#pragma unroll
  for (int k = 0; k < kNMetric; ++k) {
    const double v = block_sum(acc[k], sd);
    if (threadIdx.x == 0) w.partial[int64_t(blockIdx.x) * kNMetric + k] = v;
  }
}

__global__ __launch_bounds__(kTB) void grpo_final(GrpoArgs a, Ws w, int64_t n_blocks,
                                                  double inv_tot) {
  __shared__ double sd[kTB / kWave];
  double acc[kNMetric] = {0, 0, 0, 0, 0};
  for (int64_t b = threadIdx.x; b < n_blocks; b += kTB)
#pragma unroll
    for (int k = 0; k < kNMetric; ++k) acc[k] += w.partial[b * kNMetric + k];
#pragma unroll
  for (int k = 0; k < kNMetric; ++k) acc[k] = block_sum(acc[k], sd);
  if (threadIdx.x == 0) {
    const bool valid = w.scal[2] != 0.0;
    const float nan = __builtin_nanf("");
    a.loss[0] = valid ? float(acc[0]) : nan;   // the token weights are folded in
    if (a.metrics) {
      a.metrics[0] = valid ? float(acc[1] * inv_tot) : nan;
      a.metrics[1] = valid ? float(acc[2] * inv_tot) : nan;
      a.metrics[2] = valid ? float(acc[3] * inv_tot) : nan;
      a.metrics[3] = valid ? float(acc[4] * inv_tot) : nan;
    }
    if (a.status) a.status[0] = valid ? 0 : 1;
  }
}

}  // namespace

size_t grpo_workspace(int64_t n_tokens, int64_t n_seqs) {
  const size_t nb = size_t((n_tokens + kTB - 1) / kTB);
  return 2 * slot(size_t(n_seqs) * 8) + slot(4 * 8) + slot(nb * 8) +
         slot(nb * kNMetric * 8) + 256;
}

hipError_t launch_grpo(const GrpoArgs& a, void* workspace, hipStream_t stream) {
  const Ws w = carve(workspace, a.cu, a.n_tokens, a.n_seqs);
  hipError_t e = hipSuccess;
  const int64_t n_adv = a.advantages ? a.n_seqs : a.n_seqs / a.group_size;
  if (n_adv > 0) {
    hipLaunchKernelGGL(grpo_advantages, dim3(unsigned((n_adv + kTB - 1) / kTB)), dim3(kTB), 0,
                       stream, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(grpo_weights, dim3(1), dim3(kTB), 0, stream, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const double inv_tot = a.n_tokens > 0 ? 1.0 / double(a.n_tokens) : 0.0;
  const int64_t nb = (a.n_tokens + kTB - 1) / kTB;
  if (nb > 0 && a.correction == 1) {
    hipLaunchKernelGGL(grpo_rho_part, dim3(unsigned(nb)), dim3(kTB), 0, stream, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(grpo_rho_fold, dim3(1), dim3(kTB), 0, stream, w, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (nb > 0) {
    hipLaunchKernelGGL(grpo_tokens, dim3(unsigned(nb)), dim3(kTB), 0, stream, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(grpo_final, dim3(1), dim3(kTB), 0, stream, a, w, nb, inv_tot);
  return hipGetLastError();
}

}  // namespace rlk
