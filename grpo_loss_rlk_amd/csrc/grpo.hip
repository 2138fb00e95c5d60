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
// Three small launches: advantages (one thread per group), per-token terms
// (one thread per token, fixed 256-token blocks, per-block fp64 partial sums),
// and a single-block fixed-order fold of the partials. The token split into
// blocks depends only on T_tot, so the loss is bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace rlk {

namespace {

constexpr int kTB = 256;
constexpr int kNMetric = 5;   // sum l, clip count, TIS count, sum k3, sum rho

struct Ws {
  int64_t* cu;
  double* adv;
  double* partial;   // [n_blocks][kNMetric]
};

Ws carve(void* workspace, int64_t n_tokens, int64_t n_seqs) {
  char* p = reinterpret_cast<char*>(workspace);
  Ws w;
  w.cu = reinterpret_cast<int64_t*>(p);
  p += (size_t(n_seqs + 1) * 8 + 255) / 256 * 256;
  w.adv = reinterpret_cast<double*>(p);
  p += (size_t(n_seqs) * 8 + 255) / 256 * 256;
  w.partial = reinterpret_cast<double*>(p);
  (void)n_tokens;
  return w;
}

__global__ __launch_bounds__(kTB) void grpo_advantages(GrpoArgs a, Ws w) {
  const int64_t g = int64_t(blockIdx.x) * kTB + threadIdx.x;
  if (a.advantages) {
    if (g < a.n_seqs) {
      w.adv[g] = double(a.advantages[g]);
      if (a.adv_out) a.adv_out[g] = a.advantages[g];
    }
    return;
  }
  const int G = a.group_size;
  if (g >= a.n_seqs / G) return;
  const float* r = a.rewards + g * G;
  double mu = 0.0;
  for (int j = 0; j < G; ++j) mu += double(r[j]);
  mu /= double(G);
  double ss = 0.0;
  for (int j = 0; j < G; ++j) {
    const double d = double(r[j]) - mu;
    ss += d * d;
  }
  const double sd = sqrt(ss / double(G - a.std_ddof));
  for (int j = 0; j < G; ++j) {
    double A = double(r[j]) - mu;
    if (a.normalize_std) A /= (sd + double(a.adv_eps));
    w.adv[g * G + j] = A;
    if (a.adv_out) a.adv_out[g * G + j] = float(A);
  }
}

__global__ __launch_bounds__(kTB) void grpo_tokens(GrpoArgs a, Ws w, double inv_tot) {
  __shared__ double sd[kTB / kWave];
  const int64_t t = int64_t(blockIdx.x) * kTB + threadIdx.x;
  double acc[kNMetric] = {0, 0, 0, 0, 0};
  if (t < a.n_tokens) {
    // response owning token t: last j with cu[j] <= t (cu is non-decreasing)
    int64_t lo = 0, hi = a.n_seqs - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (w.cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const double A = w.adv[lo];
    const double C = a.tis_cap, lo_b = 1.0 - double(a.eps_low), hi_b = 1.0 + double(a.eps_high);
    const double beta = a.kl_coef;
    const double lpn = a.lp_new[t];
    const double rho = exp(lpn - double(a.lp_old[t]));
    const double rt = rho < C ? rho : C;
    const double clipped = rt < lo_b ? lo_b : (rt > hi_b ? hi_b : rt);
    const double s1 = rt * A, s2 = clipped * A;
    const double s = s1 < s2 ? s1 : s2;
    double k3 = 0.0, ed = 1.0;
    if (a.lp_ref) {
      const double delta = double(a.lp_ref[t]) - lpn;
      ed = exp(delta);
      k3 = ed - delta - 1.0;
    }
    const double ell = -s + beta * k3;
    const bool tis = rho > C;
    const bool clip = (A > 0.0 && rt > hi_b) || (A < 0.0 && rt < lo_b);
    const bool live = (rho <= C) && !(A > 0.0 && rho > hi_b) && !(A < 0.0 && rho < lo_b);
    const double g = (-(live ? A * rho : 0.0) + beta * (1.0 - ed)) * inv_tot;
    a.grad[t] = float(g);
    if (a.token_loss) a.token_loss[t] = float(ell);
    if (a.token_flags) a.token_flags[t] = uint8_t((tis ? 1 : 0) | (clip ? 2 : 0));
    acc[0] = ell;
    acc[1] = clip ? 1.0 : 0.0;
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
    a.loss[0] = float(acc[0] * inv_tot);
    if (a.metrics) {
      a.metrics[0] = float(acc[1] * inv_tot);
      a.metrics[1] = float(acc[2] * inv_tot);
      a.metrics[2] = float(acc[3] * inv_tot);
      a.metrics[3] = float(acc[4] * inv_tot);
    }
  }
}

}  // namespace

size_t grpo_workspace(int64_t n_tokens, int64_t n_seqs) {
  const size_t nb = size_t((n_tokens + kTB - 1) / kTB);
  return (size_t(n_seqs + 1) * 8 + 255) / 256 * 256 + (size_t(n_seqs) * 8 + 255) / 256 * 256 +
         (nb * kNMetric * 8 + 255) / 256 * 256 + 256;
}

hipError_t launch_grpo(const GrpoArgs& a, const int64_t* cu_host, void* workspace,
                       hipStream_t stream) {
  const Ws w = carve(workspace, a.n_tokens, a.n_seqs);
  hipError_t e = hipMemcpyAsync(w.cu, cu_host, size_t(a.n_seqs + 1) * 8, hipMemcpyHostToDevice,
                                stream);
  if (e != hipSuccess) return e;
  const int64_t n_adv = a.advantages ? a.n_seqs : a.n_seqs / a.group_size;
  if (n_adv > 0) {
    hipLaunchKernelGGL(grpo_advantages, dim3(unsigned((n_adv + kTB - 1) / kTB)), dim3(kTB), 0,
                       stream, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const double inv_tot = a.n_tokens > 0 ? 1.0 / double(a.n_tokens) : 0.0;
  const int64_t nb = (a.n_tokens + kTB - 1) / kTB;
  if (nb > 0) {
    hipLaunchKernelGGL(grpo_tokens, dim3(unsigned(nb)), dim3(kTB), 0, stream, a, w, inv_tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(grpo_final, dim3(1), dim3(kTB), 0, stream, a, w, nb, inv_tot);
  return hipGetLastError();
}

}  // namespace rlk
