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
// Work split by the size of the set only (so a row's outputs never depend on
// the batch): a block of 256 threads takes 4 rows; a row of at most 512 ids
// is scored by one wave, a larger one by the whole block afterwards. Two
// passes over the set (ids read coalesced, logits gathered, 16 loads in
// flight per thread): validation, max, min and the target; then the sums in
// fp64, each thread in index order and a fixed reduction tree. The first 16
// logits of every thread stay in registers between the passes (all of a
// wave's set), so only sets beyond 4096 ids gather anything twice.
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

constexpr int kRowsPerBlock = kST / kWave;
constexpr int64_t kWaveMaxIds = 512;   // sets up to this size are scored by one wave
// 16 ids per thread per round: the id loads and then the dependent logit
// gathers of a round are all in flight together (91 -> 81 us per 4096-row
// call against 4 per round; 32 spills and halves the occupancy)
constexpr int kU = 16;                 // ids per thread per round
constexpr int kCached = 1;             // rounds whose logits stay in registers

// Reductions over a group of G threads (a wave or the block), result in
// every thread; fixed trees.
template <int G>
struct Group;
template <>
struct Group<kWave> {
  static RLK_DEV float max(float v, float*) { return __shfl(wave_max(v), 0, kWave); }
  static RLK_DEV float min(float v, float*) { return __shfl(wave_min(v), 0, kWave); }
  static RLK_DEV int any(int v, int*) { return __any(v) ? 1 : 0; }
  static RLK_DEV double sum(double v, double*) { return __shfl(wave_sum(v), 0, kWave); }
};
template <>
struct Group<kST> {
  static RLK_DEV float max(float v, float* s) { return block_max(v, s); }
  static RLK_DEV float min(float v, float* s) { return block_min(v, s); }
  static RLK_DEV int any(int v, int* s) { return block_max(v, s); }
  static RLK_DEV double sum(double v, double* s) { return block_sum(v, s); }
};

struct Scratch {
  double d[kST / kWave];
  float f[kST / kWave];
  int i[kST / kWave];
};

// Score one row with the G threads whose index in the group is g.
template <typename T, int G>
RLK_DEV void score_row(const SupportArgs& a, int64_t row, int g, Scratch& sc) {
  using R = Group<G>;
  const int64_t V = a.vocab;
  const T* zrow = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  const int64_t y = a.targets[row];
  const int64_t o0 = a.offsets[row], o1 = a.offsets[row + 1];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  const bool range_ok = o0 >= 0 && o1 > o0 && o1 <= a.n_support;

  // ---- pass 1: ids valid and increasing, logits finite, max, min, target ----
  // The first kCached rounds keep their logits in registers for pass 2.
  int bad = range_ok ? 0 : 1, nonfin = 0, found = 0;
  float mx = -INFINITY, mn = INFINITY, zy = -INFINITY;
  float zc[kCached][kU];
  auto round1 = [&](int64_t k0, float (&z)[kU]) __attribute__((always_inline)) {
    int32_t id[kU], prev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + int64_t(u) * G;
      id[u] = k < o1 ? a.ids[k] : 0;
      prev[u] = (k < o1 && k > o0) ? a.ids[k - 1] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + int64_t(u) * G;
      const bool live = k < o1;
      const bool ok = id[u] >= 0 && id[u] < V && prev[u] < id[u];
      if (live && !ok) bad = 1;
      z[u] = (live && ok) ? value_at<T>(zrow, id[u]) : -INFINITY;
      if (live && ok) {
        if (!(fabsf(z[u]) <= 3.402823466e38f)) nonfin = 1;
        mx = fmaxf(mx, z[u]);
        mn = fminf(mn, z[u]);
        if (id[u] == y) {
          found = 1;
          zy = z[u];
        }
      }
    }
  };
  if (range_ok) {
#pragma unroll
    for (int r = 0; r < kCached; ++r) round1(o0 + g + int64_t(r) * G * kU, zc[r]);
    for (int64_t k0 = o0 + g + int64_t(kCached) * G * kU; k0 < o1; k0 += int64_t(G) * kU) {
      float z[kU];
      round1(k0, z);
    }
  }
  bad = R::any(bad, sc.i);
  nonfin = R::any(nonfin, sc.i);
  found = R::any(found, sc.i);
  mx = R::max(mx, sc.f);
  mn = R::min(mn, sc.f);
  zy = R::max(zy, sc.f);   // the only candidate is the thread that found y
  const float nan = __builtin_nanf("");
  if (bad || nonfin) {
    if (g == 0) {
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
  auto round2 = [&](int64_t k0, const float (&z)[kU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + int64_t(u) * G < o1) {
        double d;
        const double e = double(support_mass(z[u], m, c, invT, &d));
        zs += e;
        ss = fma(e, d, ss);
      }
    }
  };
#pragma unroll
  for (int r = 0; r < kCached; ++r) round2(o0 + g + int64_t(r) * G * kU, zc[r]);
  for (int64_t k0 = o0 + g + int64_t(kCached) * G * kU; k0 < o1; k0 += int64_t(G) * kU) {
    float z[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + int64_t(u) * G;
      z[u] = k < o1 ? value_at<T>(zrow, a.ids[k]) : mx;
    }
    round2(k0, z);
  }
  const double Zs = R::sum(zs, sc.d);
  const double Ss = R::sum(ss, sc.d);
  if (g != 0) return;
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

// A set is "large" when its offsets are valid and it holds more than
// kWaveMaxIds ids; everything else (including invalid ranges) is a wave's.
RLK_DEV bool large_set(const SupportArgs& a, int64_t row) {
  const int64_t o0 = a.offsets[row], o1 = a.offsets[row + 1];
  return o0 >= 0 && o1 > o0 && o1 <= a.n_support && o1 - o0 > kWaveMaxIds;
}

template <typename T>
__global__ __launch_bounds__(kST) void support_rows(SupportArgs a) {
  __shared__ Scratch sc[kRowsPerBlock + 1];
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int64_t row0 = int64_t(blockIdx.x) * kRowsPerBlock;
  {   // small sets: one wave each
    const int64_t row = row0 + w;
    if (row < a.n_rows && !large_set(a, row)) score_row<T, kWave>(a, row, lane, sc[w]);
  }
  // large sets: the whole block, one row after another
  for (int q = 0; q < kRowsPerBlock; ++q) {
    const int64_t row = row0 + q;
    if (row < a.n_rows && large_set(a, row)) score_row<T, kST>(a, row, tid, sc[kRowsPerBlock]);
  }
}

}  // namespace

hipError_t launch_support_rows(const SupportArgs& a, int dtype, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid(unsigned((a.n_rows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (dtype == 0)
    hipLaunchKernelGGL(support_rows<float>, grid, dim3(kST), 0, stream, a);
  else
    hipLaunchKernelGGL(support_rows<uint16_t>, grid, dim3(kST), 0, stream, a);
  return hipGetLastError();
}

}  // namespace rlk
