// Retained-support scoring: token log-probability and entropy over a
// caller-supplied set per row (Qwen3-8B VIME consistency page, "ROCm MI300X
// and gfx942": below top-p 1 the rollout sampler hands its complete finite
// retained-token set to the deterministic logprob kernel, which scores the
// selected token and the monitoring entropy over it; prime-rl v0.10.0
// release notes, "Breaking changes": the sampling mask travels as CSR).
//
// For row n with S = ids[offsets[n] .. offsets[n+1]): m = max_S z,
// d = (z - m)/T, Z_S = sum_S e^d, lp = d_y - log Z_S (-inf if y is not in
// S), H = log Z_S - sum_S e^d d / Z_S. A valid S is non-empty, in range,
// strictly increasing and finite. Optionally S is compared with the nucleus
// the logits-in row kernel found for the same row: S equals it exactly when
// |S| equals the nucleus size and every logit of S is >= the threshold
// (S has distinct ids, and the nucleus is {z >= tau}).
//
// One 256-thread block per row, two passes over the support (ids read
// coalesced, logits gathered): validation, max, min, target; then the sums in
// fp64 with a fixed per-thread order and a fixed block tree, so a row's
// outputs are bitwise independent of the batch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "support_kernels.h"

namespace rlk {

namespace {

constexpr int kST = 256;
constexpr uint8_t kOutside = 1, kBadTarget = 2, kNonFinite = 4, kBoundary = 8, kBadParam = 16,
                  kBadSupport = 32, kMismatch = 64;

template <typename T>
RLK_DEV float value_at(const T* row, int64_t i);
template <>
RLK_DEV float value_at<float>(const float* row, int64_t i) { return row[i]; }
template <>
RLK_DEV float value_at<uint16_t>(const uint16_t* row, int64_t i) { return bf16_to_f32(row[i]); }

// exp((z - m)/T) in fp32 to about 1 ulp: z - m exact in fp64, the exponent
// rounded once to fp32 for the hardware exp2 and its residual restored to
// first order. *d receives (z - m)/T.
RLK_DEV float support_mass(float z, double m, double c, double invT, double* d) {
  const double s = double(z) - m;
  const double x = s * c;
  const float xh = float(x);
  const float r = float(x - double(xh));
  const float e = __builtin_amdgcn_exp2f(xh);
  *d = s * invT;
  return fmaf(e, r * 0.69314718f, e);
}

template <typename T>
__global__ __launch_bounds__(kST) void support_rows(SupportArgs a) {
  __shared__ double sd[kST / kWave];
  __shared__ float sf[kST / kWave];
  __shared__ int si[kST / kWave];
  __shared__ float zy_s;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t V = a.vocab;
  const T* zrow = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  const int64_t y = a.targets[row];
  const int64_t o0 = a.offsets[row], o1 = a.offsets[row + 1];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  const bool range_ok = o0 >= 0 && o1 > o0 && o1 <= a.n_support;
  if (tid == 0) zy_s = 0.f;
  __syncthreads();

  // ---- pass 1: ids valid and increasing, logits finite, max, min, target ----
  int bad = range_ok ? 0 : 1, nonfin = 0, found = 0;
  float mx = -INFINITY, mn = INFINITY;
  if (range_ok) {
    for (int64_t k = o0 + tid; k < o1; k += kST) {
      const int32_t id = a.ids[k];
      if (id < 0 || id >= V || (k > o0 && a.ids[k - 1] >= id)) {
        bad = 1;
        continue;
      }
      const float z = value_at<T>(zrow, id);
      if (!(fabsf(z) <= 3.402823466e38f)) nonfin = 1;
      mx = fmaxf(mx, z);
      mn = fminf(mn, z);
      if (id == y) {
        found = 1;
        zy_s = z;
      }
    }
  }
  __syncthreads();
  bad = block_max(bad, si);
  nonfin = block_max(nonfin, si);
  found = block_max(found, si);
  mx = block_max(mx, sf);
  mn = block_min(mn, sf);
  const float zy = zy_s;
  const float nan = __builtin_nanf("");
  if (bad || nonfin) {
    if (tid == 0) {
      a.lp[row] = nan;
      a.ent[row] = nan;
      if (a.flags) a.flags[row] = flags | (bad ? kBadSupport : kNonFinite);
    }
    return;
  }

  // ---- pass 2: Z_S and sum e d over S in fp64, fixed order ----
  const double m = double(mx), invT = 1.0 / double(a.temperature);
  const double c = 1.4426950408889634 * invT;
  double zs = 0.0, ss = 0.0;
  for (int64_t k = o0 + tid; k < o1; k += kST) {
    double d;
    const double e = double(support_mass(value_at<T>(zrow, a.ids[k]), m, c, invT, &d));
    zs += e;
    ss = fma(e, d, ss);
  }
  const double Zs = block_sum(zs, sd);
  const double Ss = block_sum(ss, sd);
  if (tid != 0) return;
  const double logZs = log(Zs);
  float lp = nan;
  if (!(flags & kBadTarget)) {
    if (found) {
      lp = float((double(zy) - m) * invT - logZs);
    } else {
      lp = -INFINITY;
      flags |= kOutside;
    }
  }
  if (a.nsize) {   // compare with the recomputed nucleus of the row
    const uint8_t nf = a.nflags[row];
    if (!(nf & (kNonFinite | kBadParam))) {
      if (nf & kBoundary) flags |= kBoundary;
      if (int64_t(a.nsize[row]) != o1 - o0 || mn < a.thresh[row]) flags |= kMismatch;
    }
  }
  a.lp[row] = lp;
  a.ent[row] = float(logZs - Ss / Zs);
  if (a.flags) a.flags[row] = flags;
}

}  // namespace

hipError_t launch_support_rows(const SupportArgs& a, int dtype, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_rows));
  if (dtype == 0)
    hipLaunchKernelGGL(support_rows<float>, grid, dim3(kST), 0, stream, a);
  else
    hipLaunchKernelGGL(support_rows<uint16_t>, grid, dim3(kST), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
