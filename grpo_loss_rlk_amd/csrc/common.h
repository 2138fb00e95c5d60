// Internal helpers shared by the rlk HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#define RLK_DEV __device__ __forceinline__

namespace rlk {

constexpr int kWave = 64;

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

}  // namespace rlk
