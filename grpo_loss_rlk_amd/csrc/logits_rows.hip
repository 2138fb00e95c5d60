// Logits in: full and top-p truncated log-probability and entropy per row.
//
// What is computed (Qwen3-8B VIME train-rollout consistency page, "ROCm MI300X
// and gfx942": temperature > 0, top-p in (0, 1], the complete nucleus is
// scored, top-p = 1 is the full vocabulary, a monitoring entropy is fused
// with the logprob): for a row z, d_i = (z_i - max z)/T, the full softmax
// statistics, the nucleus S = {z >= tau} with tau the lowest row value whose
// strictly-higher mass is below p (all ties kept), and the statistics of the
// distribution renormalised over S.
//
// Two kernels, chosen per call by dtype and vocabulary size only (never by the
// number of rows, so a row's result does not depend on its batch):
//
//  * bf16_hist_rows: bf16 rows with V >= 16384. A bf16 value has only 65536
//    bit patterns, so one streaming pass that counts each pattern in LDS
//    (16-bit counters, two per 32-bit word, 128 KB) captures the whole row.
//    Everything after that -- max, Z, entropy, the top-p cut, the truncated
//    sums -- is exact arithmetic over the distinct values (fp64, fixed
//    order), so HBM is read once at 5 VALU ops per element. A 16-bit counter
//    that would exceed 65535 (one value holding > 43% of a long row) is
//    detected by a checksum and the row is handed to the generic kernel.
//
//  * generic_rows: any dtype and size. Multi-pass over the row: max, then
//    exp / Z / entropy with a 12-bit radix histogram of fixed-point masses,
//    then two refinement rounds (10 + 10 bits) restricted to the boundary
//    bin, then the truncated sums. Masses are integers (2^-39 of the max
//    element's mass) so LDS atomics are order-free and the cut is bitwise
//    deterministic.
#include "common.h"
#include "kernels.h"

namespace rlk {

namespace {

constexpr uint8_t kOutside = 1, kBadTarget = 2, kNonFinite = 4, kBoundary = 8, kBadParam = 16;
constexpr double kBoundaryEps = 1e-6;

RLK_DEV bool param_ok(float T, float p) {
  return T > 0.f && T <= 3.4e38f && p > 0.f && p <= 1.f;  // NaN fails every compare
}

RLK_DEV void store_row(const RowArgs& a, int64_t row, float lp_full, float lp_trunc,
                       float h_full, float h_trunc, int32_t size, float tau, uint8_t flags) {
  a.lp_full[row] = lp_full;
  a.lp_trunc[row] = lp_trunc;
  a.ent_trunc[row] = h_trunc;
  if (a.ent_full) a.ent_full[row] = h_full;
  if (a.nsize) a.nsize[row] = size;
  if (a.thresh) a.thresh[row] = tau;
  if (a.flags) a.flags[row] = flags;
}

RLK_DEV void store_nan_row(const RowArgs& a, int64_t row, uint8_t flags) {
  const float nan = __builtin_nanf("");
  store_row(a, row, nan, nan, nan, nan, 0, nan, flags);
}

// ===========================================================================
// bf16 pattern-count histogram kernel
// ===========================================================================
constexpr int kHT = 1024;              // threads per row
constexpr int kHWords = 32768;         // word w: lo16 = count(code w), hi16 = count(code 0x8000|w)
constexpr int kWordsPerThread = kHWords / kHT;
constexpr uint32_t kInfW = 0x7f80;     // codes with w >= 0x7f80 are inf / NaN

RLK_DEV void hist_add(uint32_t* hist, uint32_t code) {
  atomicAdd(&hist[code & 0x7fffu], (code & 0x8000u) ? 0x10000u : 1u);
}

// Merged key order over bf16 patterns: key = code | 0x8000 for positive codes,
// ~code & 0xffff for negative ones; -0 (key 0x7fff) is folded into +0 (0x8000).
// Returns the count of the value with this key, and the value.
RLK_DEV uint32_t key_count(const uint32_t* hist, uint32_t key, float* value) {
  if (key >= 0x8000u) {
    const uint32_t c = key - 0x8000u;
    uint32_t n = hist[c] & 0xffffu;
    if (c == 0) n += hist[0] >> 16;   // -0 joins +0
    *value = bf16_to_f32(uint16_t(c));
    return n;
  }
  const uint32_t c = (~key) & 0xffffu;   // negative code
  *value = bf16_to_f32(uint16_t(c));
  if (c == 0x8000u) return 0;            // -0 already counted with +0
  return hist[c & 0x7fffu] >> 16;
}

RLK_DEV uint32_t bf16_key_merged(uint16_t code) {
  if (code == 0x8000u) code = 0;
  return (code & 0x8000u) ? ((~uint32_t(code)) & 0xffffu) : (uint32_t(code) | 0x8000u);
}

template <bool kVec>
__global__ __launch_bounds__(kHT) void bf16_hist_rows(RowArgs a) {
  __shared__ uint32_t hist[kHWords];
  __shared__ double sd[kHT / kWave], sd2[kHT / kWave];
  __shared__ int si[kHT / kWave];
  __shared__ uint32_t su[kHT / kWave];
  __shared__ double bcast_d[3];
  __shared__ int bcast_i[1];

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t V = a.vocab;
  const uint16_t* rowp = reinterpret_cast<const uint16_t*>(a.logits) + row * a.row_stride;

  // the target's logit is fetched early so its latency hides behind the pass
  const int64_t y = a.targets[row];
  const bool y_ok = y >= 0 && y < V;
  uint16_t cy = 0;
  if (tid == 0 && y_ok) cy = rowp[y];

  {  // clear the histogram
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (int i = tid; i < kHWords / 4; i += kHT) h4[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // ---- one streaming pass: count every bf16 pattern of the row ----
  if (kVec) {
    const uint4* v4 = reinterpret_cast<const uint4*>(rowp);
    const int64_t nvec = V >> 3;
    int64_t i = tid;
    for (; i + 3 * kHT < nvec; i += 4 * kHT) {
      uint4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = v4[i + u * kHT];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        hist_add(hist, q[u].x & 0xffffu); hist_add(hist, q[u].x >> 16);
        hist_add(hist, q[u].y & 0xffffu); hist_add(hist, q[u].y >> 16);
        hist_add(hist, q[u].z & 0xffffu); hist_add(hist, q[u].z >> 16);
        hist_add(hist, q[u].w & 0xffffu); hist_add(hist, q[u].w >> 16);
      }
    }
    for (; i < nvec; i += kHT) {
      const uint4 q = v4[i];
      hist_add(hist, q.x & 0xffffu); hist_add(hist, q.x >> 16);
      hist_add(hist, q.y & 0xffffu); hist_add(hist, q.y >> 16);
      hist_add(hist, q.z & 0xffffu); hist_add(hist, q.z >> 16);
      hist_add(hist, q.w & 0xffffu); hist_add(hist, q.w >> 16);
    }
    for (int64_t j = (nvec << 3) + tid; j < V; j += kHT) hist_add(hist, rowp[j]);
  } else {
    for (int64_t j = tid; j < V; j += kHT) hist_add(hist, rowp[j]);
  }
  __syncthreads();

  // ---- checksum, max and non-finite detection over the counters ----
  uint32_t tot = 0, n_neg_inf = 0;
  int maxpos = -1, minneg = 0x8000, nonfinite = 0;
  for (int j = 0; j < kWordsPerThread; ++j) {
    const int w = tid + j * kHT;
    const uint32_t x = hist[w];
    const uint32_t lo = x & 0xffffu, hi = x >> 16;
    tot += lo + hi;
    if (w < int(kInfW)) {
      if (lo) maxpos = w;
      if (hi && w < minneg) minneg = w;
    } else {
      if (lo) nonfinite = 1;                         // +inf or NaN
      if (hi && w > int(kInfW)) nonfinite = 1;       // NaN
      if (w == int(kInfW)) n_neg_inf = hi;           // -inf
    }
  }
  tot = block_sum(tot, su);
  maxpos = block_max(maxpos, si);
  minneg = block_min(minneg, si);
  nonfinite = block_max(nonfinite, si);
  n_neg_inf = block_sum(n_neg_inf, su);

  if (tot != uint32_t(V)) {          // a 16-bit counter overflowed: generic kernel
    if (tid == 0) a.fallback[row] = 1;
    return;
  }

  float T = a.t_row ? a.t_row[row] : a.temperature;
  float p = a.p_row ? a.p_row[row] : a.top_p;
  uint8_t flags = 0;
  if (!y_ok) flags |= kBadTarget;
  if (!param_ok(T, p)) flags |= kBadParam;
  const bool no_finite = (maxpos < 0 && minneg == 0x8000);
  if (nonfinite || no_finite) flags |= kNonFinite;
  if (flags & (kNonFinite | kBadParam)) {
    if (tid == 0) {
      a.fallback[row] = 0;
      store_nan_row(a, row, flags);
    }
    return;
  }

  // max value and its merged key
  float mval;
  uint32_t kmax;
  if (maxpos >= 0) {
    mval = bf16_to_f32(uint16_t(maxpos));
    kmax = 0x8000u + uint32_t(maxpos);
  } else if (minneg == 0) {          // only -0 at the top: same value as +0
    mval = 0.f;
    kmax = 0x8000u;
  } else {
    mval = bf16_to_f32(uint16_t(0x8000 | minneg));
    kmax = 0x7fffu - uint32_t(minneg);
  }
  const double m = double(mval);
  const double invT = 1.0 / double(T);

  // ---- Z and sum e*d over the distinct finite values (fp64) ----
  double zt = 0.0, st = 0.0;
  for (int j = 0; j < kWordsPerThread; ++j) {
    const int w = tid + j * kHT;
    if (w >= int(kInfW)) break;
    const uint32_t x = hist[w];
    const uint32_t lo = x & 0xffffu, hi = x >> 16;
    if (lo) {
      const double d = (double(bf16_to_f32(uint16_t(w))) - m) * invT;
      const double e = exp(d) * double(lo);
      zt += e;
      st += e * d;
    }
    if (hi) {
      const double d = (double(bf16_to_f32(uint16_t(0x8000 | w))) - m) * invT;
      const double e = exp(d) * double(hi);
      zt += e;
      st += e * d;
    }
  }
  const double Z = block_sum(zt, sd);
  const double S = block_sum(st, sd);

  // ---- top-p cut: walk merged keys downward from the max ----
  double Zs = Z, Ss = S, Mgt = 0.0;
  uint32_t tau_key = 0;
  const bool cut = p < 1.f;
  if (cut) {
    const double thr = double(p) * Z;
    double carry = 0.0, carry_s = 0.0;
    bool found = false;
    for (int k0 = int(kmax); k0 >= 0x0080 && !found; k0 -= kHT) {
      const int key = k0 - tid;
      double mass = 0.0, mass_s = 0.0;
      if (key >= 0x0080) {                      // keys below 0x0080 are -inf / NaN
        float v;
        const uint32_t n = key_count(hist, uint32_t(key), &v);
        if (n) {
          const double d = (double(v) - m) * invT;
          mass = exp(d) * double(n);
          mass_s = mass * d;
        }
      }
      double tot_c, tot_s;
      const double incl = block_inclusive_scan(mass, sd, &tot_c);
      const double incl_s = block_inclusive_scan(mass_s, sd2, &tot_s);
      const int cand = (mass > 0.0 && carry + incl >= thr) ? tid : kHT;
      const int first = block_min(cand, si);
      if (first < kHT) {
        if (tid == first) {
          bcast_d[0] = carry + incl;
          bcast_d[1] = carry_s + incl_s;
          bcast_d[2] = carry + incl - mass;
          bcast_i[0] = key;
        }
        __syncthreads();
        Zs = bcast_d[0];
        Ss = bcast_d[1];
        Mgt = bcast_d[2];
        tau_key = uint32_t(bcast_i[0]);
        found = true;
      } else {
        carry += tot_c;
        carry_s += tot_s;
      }
    }
    if (!found) {   // rounding left the mass just short of p: keep every finite value
      Zs = carry;
      Ss = carry_s;
      Mgt = carry;
      tau_key = 0x0080;
    }
  }

  // ---- |S| ----
  uint32_t size;
  if (cut) {
    uint32_t cnt = 0;
    for (int j = 0; j < kWordsPerThread; ++j) {
      const int w = tid + j * kHT;
      if (w >= int(kInfW)) break;
      const uint32_t x = hist[w];
      if (0x8000u + uint32_t(w) >= tau_key) cnt += x & 0xffffu;
      const uint32_t kneg = (w == 0) ? 0x8000u : 0x7fffu - uint32_t(w);  // -0 merged into +0
      if (kneg >= tau_key) cnt += x >> 16;
    }
    size = block_sum(cnt, su);
  } else {
    size = uint32_t(V) - n_neg_inf;
  }

  if (tid == 0) {
    a.fallback[row] = 0;
    const double logZ = log(Z), logZs = log(Zs);
    const float h_full = float(logZ - S / Z);
    const float h_trunc = float(logZs - Ss / Zs);
    float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
    if (!(flags & kBadTarget)) {
      const float vy = bf16_to_f32(cy);
      if (vy == -INFINITY) {
        lpf = -INFINITY;
        lpt = -INFINITY;
        flags |= kOutside;
      } else {
        const double dy = (double(vy) - m) * invT;
        lpf = float(dy - logZ);
        if (!cut || bf16_key_merged(cy) >= tau_key) {
          lpt = float(dy - logZs);
        } else {
          lpt = -INFINITY;
          flags |= kOutside;
        }
      }
    }
    float tau = -INFINITY;
    if (cut) {
      float tv;
      key_count(hist, tau_key, &tv);
      tau = (tau_key == 0x8000u) ? 0.f : tv;
      const double pp = double(p);
      if (fabs(Mgt / Z - pp) <= kBoundaryEps || fabs(Zs / Z - pp) <= kBoundaryEps) flags |= kBoundary;
    }
    store_row(a, row, lpf, lpt, h_full, h_trunc, int32_t(size), tau, flags);
  }
}

// ===========================================================================
// Generic radix-select kernel (fp32 or bf16 rows of any length)
// ===========================================================================
constexpr int kGT = 256;
constexpr int kBins1 = 4096;          // round 1: top 12 key bits
constexpr int kBins2 = 1024;          // rounds 2, 3: 10 bits each
constexpr double kFix = 549755813888.0;   // 2^39: fixed-point unit of mass (max element = 2^39)

template <typename T>
RLK_DEV float load_val(const T* p, int64_t i);
template <>
RLK_DEV float load_val<float>(const float* p, int64_t i) { return p[i]; }
template <>
RLK_DEV float load_val<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// exp((z - m) / T) in fp32 from an fp64 argument, and d = (z - m)/T in fp64
RLK_DEV float mass_of(float z, double m, double invT, double* d) {
  *d = (double(z) - m) * invT;
  return expf(float(*d));
}

RLK_DEV uint64_t fixed_mass(float e) { return uint64_t(double(e) * kFix + 0.5); }

// Walk `bins` from index `start` downward until carry + running sum >= thr.
// Returns the bin, or -1; *above receives the mass strictly above that bin.
RLK_DEV int walk_down(const uint64_t* bins, int start, uint64_t thr, uint64_t carry,
                      uint64_t* above, uint64_t* su64, int* si, uint64_t* bslot) {
  for (int base = start; base >= 0; base -= kGT) {
    const int b = base - int(threadIdx.x);
    const uint64_t v = b >= 0 ? bins[b] : 0ull;
    uint64_t tot;
    const uint64_t incl = block_inclusive_scan(v, su64, &tot);
    const int cand = (v != 0ull && carry + incl >= thr) ? int(threadIdx.x) : kGT;
    const int first = block_min(cand, si);
    if (first < kGT) {
      if (int(threadIdx.x) == first) *bslot = carry + incl - v;
      __syncthreads();
      *above = *bslot;
      __syncthreads();
      return base - first;
    }
    carry += tot;
  }
  *above = carry;
  return -1;
}

template <typename T>
__global__ __launch_bounds__(kGT) void generic_rows(RowArgs a, int only_fallback) {
  __shared__ uint64_t hist[kBins1];
  __shared__ double sd[kGT / kWave];
  __shared__ uint64_t su64[kGT / kWave];
  __shared__ int si[kGT / kWave];
  __shared__ float sf[kGT / kWave];
  __shared__ uint64_t bslot;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (only_fallback && a.fallback[row] == 0) return;
  const int64_t V = a.vocab;
  const T* rowp = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;

  float Tv = a.t_row ? a.t_row[row] : a.temperature;
  float p = a.p_row ? a.p_row[row] : a.top_p;
  const int64_t y = a.targets[row];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  if (!param_ok(Tv, p)) {
    if (tid == 0) store_nan_row(a, row, flags | kBadParam);
    return;
  }

  // ---- pass 1: max, finite count, non-finite detection ----
  float mx = -INFINITY;
  int bad = 0;
  uint32_t nfin = 0;
  for (int64_t i = tid; i < V; i += kGT) {
    const float z = load_val(rowp, i);
    if (z != z || z == INFINITY) bad = 1;
    else if (z > -INFINITY) {
      mx = fmaxf(mx, z);
      ++nfin;
    }
  }
  mx = block_max(mx, sf);
  bad = block_max(bad, si);
  nfin = uint32_t(block_sum(uint64_t(nfin), su64));
  if (bad || nfin == 0) {
    if (tid == 0) store_nan_row(a, row, flags | kNonFinite);
    return;
  }
  const double m = double(mx);
  const double invT = 1.0 / double(Tv);
  const bool cut = p < 1.f;

  // ---- pass 2: Z, sum e*d, round-1 histogram of fixed-point masses ----
  for (int i = tid; i < kBins1; i += kGT) hist[i] = 0ull;
  __syncthreads();
  double zt = 0.0, st = 0.0;
  uint64_t wt = 0;
  for (int64_t i = tid; i < V; i += kGT) {
    const float z = load_val(rowp, i);
    if (!(z > -INFINITY)) continue;
    double d;
    const float e = mass_of(z, m, invT, &d);
    zt += double(e);
    st += double(e) * d;
    if (cut) {
      const uint64_t w = fixed_mass(e);
      if (w) {
        wt += w;
        atomicAdd(reinterpret_cast<unsigned long long*>(&hist[f32_key(z) >> 20]),
                  (unsigned long long)w);
      }
    }
  }
  const double Z = block_sum(zt, sd);
  const double S = block_sum(st, sd);

  double Zs = Z, Ss = S;
  uint32_t tau_key = 0;
  uint32_t size = nfin;
  if (cut) {
    const uint64_t W = block_sum(wt, su64);
    const uint64_t thr = uint64_t(ceil(double(p) * double(W)));
    // round 1
    uint64_t above = 0;
    int d1 = walk_down(hist, kBins1 - 1, thr, 0ull, &above, su64, si, &bslot);
    if (d1 < 0) d1 = 0;   // unreachable: the total mass reaches thr
    // round 2
    __syncthreads();
    for (int i = tid; i < kBins2; i += kGT) hist[i] = 0ull;
    __syncthreads();
    for (int64_t i = tid; i < V; i += kGT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = f32_key(z);
      if (int(k >> 20) != d1) continue;
      double d;
      const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
      if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(k >> 10) & 0x3ffu]),
                       (unsigned long long)w);
    }
    __syncthreads();
    int d2 = walk_down(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
    if (d2 < 0) d2 = 0;
    // round 3
    __syncthreads();
    for (int i = tid; i < kBins2; i += kGT) hist[i] = 0ull;
    __syncthreads();
    const uint32_t pre = (uint32_t(d1) << 10) | uint32_t(d2);
    for (int64_t i = tid; i < V; i += kGT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = f32_key(z);
      if ((k >> 10) != pre) continue;
      double d;
      const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
      if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[k & 0x3ffu]),
                       (unsigned long long)w);
    }
    __syncthreads();
    int d3 = walk_down(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
    if (d3 < 0) d3 = 0;
    tau_key = (pre << 10) | uint32_t(d3);
    const uint64_t at = hist[d3];
    if (tid == 0) {
      const double pp = double(p);
      if (fabs(double(above) / double(W) - pp) <= kBoundaryEps ||
          fabs(double(above + at) / double(W) - pp) <= kBoundaryEps)
        flags |= kBoundary;
    }
    // final pass: truncated sums over S = {key >= tau}
    double zs = 0.0, ss = 0.0;
    uint32_t cnt = 0;
    for (int64_t i = tid; i < V; i += kGT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY) || f32_key(z) < tau_key) continue;
      double d;
      const float e = mass_of(z, m, invT, &d);
      zs += double(e);
      ss += double(e) * d;
      ++cnt;
    }
    Zs = block_sum(zs, sd);
    Ss = block_sum(ss, sd);
    size = uint32_t(block_sum(uint64_t(cnt), su64));
  }

  if (tid == 0) {
    const double logZ = log(Z), logZs = log(Zs);
    float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
    if (!(flags & kBadTarget)) {
      const float zy = load_val(rowp, y);
      if (!(zy > -INFINITY)) {
        lpf = -INFINITY;
        lpt = -INFINITY;
        flags |= kOutside;
      } else {
        const double dy = (double(zy) - m) * invT;
        lpf = float(dy - logZ);
        if (!cut || f32_key(zy) >= tau_key) {
          lpt = float(dy - logZs);
        } else {
          lpt = -INFINITY;
          flags |= kOutside;
        }
      }
    }
    const float tau = cut ? key_f32(tau_key) : -INFINITY;
    store_row(a, row, lpf, lpt, float(logZ - S / Z), float(logZs - Ss / Zs), int32_t(size), tau,
              flags);
  }
}

}  // namespace

size_t logits_rows_workspace(int64_t n_rows, int64_t vocab, int dtype) {
  (void)vocab;
  (void)dtype;
  return size_t((n_rows + 255) / 256 * 256);
}

hipError_t launch_logits_rows(const RowArgs& a, int dtype, void* workspace, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  RowArgs args = a;
  args.fallback = reinterpret_cast<uint8_t*>(workspace);
  const dim3 grid(unsigned(a.n_rows));
  if (dtype == 0) {  // fp32
    hipLaunchKernelGGL(generic_rows<float>, grid, dim3(kGT), 0, stream, args, 0);
    return hipGetLastError();
  }
  if (a.vocab < 16384) {
    hipLaunchKernelGGL(generic_rows<uint16_t>, grid, dim3(kGT), 0, stream, args, 0);
    return hipGetLastError();
  }
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 8 == 0);
  if (vec)
    hipLaunchKernelGGL(bf16_hist_rows<true>, grid, dim3(kHT), 0, stream, args);
  else
    hipLaunchKernelGGL(bf16_hist_rows<false>, grid, dim3(kHT), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.vocab > 65535) {   // a 16-bit counter can only overflow in rows this long
    hipLaunchKernelGGL(generic_rows<uint16_t>, grid, dim3(kGT), 0, stream, args, 1);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace rlk
