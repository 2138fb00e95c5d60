// Internal helpers shared by the rlk HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <cmath>

#define RLK_DEV __device__ __forceinline__

namespace rlk {

constexpr int kWave = 64;

// Log-probability of a token with logit zy in a row whose max is m and whose
// log-normaliser (over the nucleus, or the whole row) is logZ, on the scale
// z/T after subtracting m: (zy - m) / T - logZ in fp64, rounded to fp32. The
// fp64 operations are rounded one by one (no contraction into a fused
// multiply-add), so every kernel that scores a token from the same (m, logZ)
// returns the same bits.
RLK_DEV float token_logprob(float zy, double m, double invT, double logZ) {
#pragma clang fp contract(off)
  const double d = (double(zy) - m) * invT;
  return float(d - logZ);
}

// Order-preserving 32-bit key of an fp32 value: a < b  <=>  key(a) < key(b)
// for non-NaN values, with -0 folded onto +0 so that equal values share a key.
RLK_DEV uint32_t f32_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

RLK_DEV float key_f32(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

RLK_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// ---------------------------------------------------------------------------
// Fixed-order block reductions. Each wave reduces with a shuffle-down tree
// (lane 0 holds the result), then wave 0 folds the per-wave partials in wave
// order. The result is returned to every thread. The order of additions is a
// function of blockDim only, so results are bitwise reproducible.
// `scratch` must hold one T per wave; the call contains two barriers.
// ---------------------------------------------------------------------------
template <typename T>
RLK_DEV T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_down(v, off, kWave);
  return v;
}

template <typename T>
RLK_DEV T wave_max(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    T o = __shfl_down(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

template <typename T>
RLK_DEV T wave_min(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    T o = __shfl_down(v, off, kWave);
    v = o < v ? o : v;
  }
  return v;
}

template <typename T>
RLK_DEV T block_sum(T v, T* scratch) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  v = wave_sum(v);
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  T r = T(0);
  for (int w = 0; w < nw; ++w) r += scratch[w];
  __syncthreads();
  return r;
}

template <typename T>
RLK_DEV T block_max(T v, T* scratch) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  v = wave_max(v);
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  T r = scratch[0];
  for (int w = 1; w < nw; ++w) r = scratch[w] > r ? scratch[w] : r;
  __syncthreads();
  return r;
}

template <typename T>
RLK_DEV T block_min(T v, T* scratch) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  v = wave_min(v);
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  T r = scratch[0];
  for (int w = 1; w < nw; ++w) r = scratch[w] < r ? scratch[w] : r;
  __syncthreads();
  return r;
}

// Inclusive prefix sum over the block in thread order (fixed order: a
// Hillis-Steele scan inside each wave, then a serial scan over wave totals).
// Returns the inclusive prefix; *total receives the block total.
template <typename T>
RLK_DEV T block_inclusive_scan(T v, T* scratch, T* total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    T o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) scratch[wid] = v;
  __syncthreads();
  T base = T(0), tot = T(0);
  for (int w = 0; w < nw; ++w) {
    if (w == wid) base = tot;
    tot += scratch[w];
  }
  __syncthreads();
  *total = tot;
  return base + v;
}

// ---------------------------------------------------------------------------
// DPP wave primitives (gfx9 data-parallel primitives: row_shr / row_bcast).
// Register-to-register lane moves with no LDS traffic. Fixed lane order, so
// floating-point results are bitwise reproducible.
// ---------------------------------------------------------------------------
template <int kCtrl, int kRowMask = 0xf, int kBankMask = 0xf>
RLK_DEV uint32_t dpp_u32(uint32_t fill, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(fill), int(v), kCtrl, kRowMask, kBankMask, false));
}

template <int kCtrl, int kRowMask = 0xf, int kBankMask = 0xf>
RLK_DEV double dpp_f64(double fill, double v) {
  const uint64_t f = __double_as_longlong(fill), x = __double_as_longlong(v);
  const uint32_t lo = dpp_u32<kCtrl, kRowMask, kBankMask>(uint32_t(f), uint32_t(x));
  const uint32_t hi = dpp_u32<kCtrl, kRowMask, kBankMask>(uint32_t(f >> 32), uint32_t(x >> 32));
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

template <int kCtrl, int kRowMask = 0xf, int kBankMask = 0xf>
RLK_DEV uint64_t dpp_u64(uint64_t fill, uint64_t v) {
  const uint32_t lo = dpp_u32<kCtrl, kRowMask, kBankMask>(uint32_t(fill), uint32_t(v));
  const uint32_t hi = dpp_u32<kCtrl, kRowMask, kBankMask>(uint32_t(fill >> 32), uint32_t(v >> 32));
  return (uint64_t(hi) << 32) | lo;
}

template <int kCtrl, int kRowMask = 0xf, int kBankMask = 0xf>
RLK_DEV float dpp_f32(float fill, float v) {
  return __uint_as_float(dpp_u32<kCtrl, kRowMask, kBankMask>(__float_as_uint(fill), __float_as_uint(v)));
}

template <int kCtrl, int kRowMask = 0xf, int kBankMask = 0xf>
RLK_DEV int dpp_i32(int fill, int v) {
  return int(dpp_u32<kCtrl, kRowMask, kBankMask>(uint32_t(fill), uint32_t(v)));
}

// Inclusive scan (sum) across the 64 lanes of a wave; lane i gets sum of lanes 0..i.
#define RLK_DPP_SCAN(T, MOVE)                                            \
  RLK_DEV T wave_scan_incl(T v) {                                        \
    v += MOVE<0x111>(T(0), v);             /* row_shr:1 */              \
    v += MOVE<0x112>(T(0), v);             /* row_shr:2 */              \
    v += MOVE<0x114>(T(0), v);             /* row_shr:4 */              \
    v += MOVE<0x118>(T(0), v);             /* row_shr:8 */              \
    v += MOVE<0x142, 0xa>(T(0), v);        /* row_bcast:15 -> rows 1,3 */ \
    v += MOVE<0x143, 0xc>(T(0), v);        /* row_bcast:31 -> rows 2,3 */ \
    return v;                                                            \
  }
RLK_DPP_SCAN(double, dpp_f64)
RLK_DPP_SCAN(float, dpp_f32)
RLK_DPP_SCAN(int, dpp_i32)
RLK_DPP_SCAN(uint64_t, dpp_u64)
#undef RLK_DPP_SCAN

RLK_DEV uint32_t readlane_u32(uint32_t v, int lane) {
  return uint32_t(__builtin_amdgcn_readlane(int(v), lane));
}
RLK_DEV double readlane_f64(double v, int lane) {
  const uint64_t x = __double_as_longlong(v);
  const uint32_t lo = readlane_u32(uint32_t(x), lane), hi = readlane_u32(uint32_t(x >> 32), lane);
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

RLK_DEV uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = readlane_u32(uint32_t(v), lane), hi = readlane_u32(uint32_t(v >> 32), lane);
  return (uint64_t(hi) << 32) | lo;
}

// Wave totals via the inclusive scan's last lane (uniform result).
RLK_DEV double wave_total(double v) { return readlane_f64(wave_scan_incl(v), kWave - 1); }
RLK_DEV int wave_total(int v) { return int(readlane_u32(uint32_t(wave_scan_incl(v)), kWave - 1)); }
RLK_DEV uint64_t wave_total(uint64_t v) { return readlane_u64(wave_scan_incl(v), kWave - 1); }

// Exclusive scan from an inclusive one: lane i gets lane i-1's value (lane 0: 0).
RLK_DEV double wave_shift_up(double v) { return dpp_f64<0x138>(0.0, v); }   // wave_shr:1
RLK_DEV int wave_shift_up(int v) { return dpp_i32<0x138>(0, v); }
RLK_DEV uint64_t wave_shift_up(uint64_t v) { return dpp_u64<0x138>(uint64_t(0), v); }

// Fold of per-wave partials p[0..n) (n <= 64) held in LDS: lane w loads p[w]
// and the wave reduces with DPP. Uniform result, fixed order.
RLK_DEV double fold_partials(const double* p, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  return wave_total(lane < n ? p[lane] : 0.0);
}
RLK_DEV int fold_partials(const int* p, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  return wave_total(lane < n ? p[lane] : 0);
}
RLK_DEV uint64_t fold_partials(const uint64_t* p, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  return wave_total(lane < n ? p[lane] : uint64_t(0));
}

// Wave max / min of ints (uniform result).
RLK_DEV int wave_max_i32(int v) {
#define RLK_STEP(C, RM) { const int o = dpp_i32<C, RM>(INT_MIN, v); v = o > v ? o : v; }
  RLK_STEP(0x111, 0xf) RLK_STEP(0x112, 0xf) RLK_STEP(0x114, 0xf) RLK_STEP(0x118, 0xf)
  RLK_STEP(0x142, 0xa) RLK_STEP(0x143, 0xc)
#undef RLK_STEP
  return int(readlane_u32(uint32_t(v), kWave - 1));
}
RLK_DEV int wave_min_i32(int v) {
#define RLK_STEP(C, RM) { const int o = dpp_i32<C, RM>(INT_MAX, v); v = o < v ? o : v; }
  RLK_STEP(0x111, 0xf) RLK_STEP(0x112, 0xf) RLK_STEP(0x114, 0xf) RLK_STEP(0x118, 0xf)
  RLK_STEP(0x142, 0xa) RLK_STEP(0x143, 0xc)
#undef RLK_STEP
  return int(readlane_u32(uint32_t(v), kWave - 1));
}

}  // namespace rlk
