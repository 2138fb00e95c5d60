// Top-p sampler on the logits-in row kernel (the rollout side of the replay:
// prime-rl v0.10.0 release notes, "2. RL Algorithms", top-p sampling is
// replayed exactly in the trainer; the consistency page requires bitwise
// agreement between rollout and training logprobs).
//
// After the row kernel has found each row's nucleus threshold tau, one block
// per row draws y = argmax over {z_i >= tau} of z_i / T - log(-log u_i), the
// lowest id on an exact tie, with u_i from Philox-4x32-10 (Salmon, Moraes,
// Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011):
// counter (i / 4, row key low, row key high, offset), key (seed low, seed
// high), word i % 4, u = (word + 1/2) 2^-32. The scores are fp64. The draw
// depends on the row, the seed, the offset and the row key only.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "sampler_kernels.h"

namespace rlk {

namespace {

constexpr int kSmT = 256;
constexpr uint8_t kNonFinite = 4, kBadParam = 16;

// Ten Philox-4x32 rounds on counter c with key (k0, k1).
RLK_DEV void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c[0]), lo0 = kM0 * c[0];
    const uint32_t hi1 = __umulhi(kM1, c[2]), lo1 = kM1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

template <typename T>
RLK_DEV float val(const T* row, int64_t i);
template <>
RLK_DEV float val<float>(const float* row, int64_t i) { return row[i]; }
template <>
RLK_DEV float val<uint16_t>(const uint16_t* row, int64_t i) { return bf16_to_f32(row[i]); }

// (score, id) order: higher score first, then the lower id
RLK_DEV bool better(double s, int64_t i, double s2, int64_t i2) {
  return s > s2 || (s == s2 && i < i2);
}

template <typename T>
__global__ __launch_bounds__(kSmT) void sample_rows(SampleArgs a) {
  __shared__ double ss[kSmT / kWave];
  __shared__ int64_t si[kSmT / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t row = blockIdx.x;
  if (a.nflags[row] & (kNonFinite | kBadParam)) {
    if (tid == 0) a.samples[row] = -1;
    return;
  }
  const T* zrow = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  const int64_t V = a.vocab;
  const float tau = a.thresh[row];
  const double T64 = double(a.temperature);
  const uint64_t rk = a.row_keys ? uint64_t(a.row_keys[row]) : uint64_t(row);
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  double best = -INFINITY;
  int64_t best_i = INT64_MAX;
  // thread t takes groups of 4 consecutive ids t, t + 256, ... (one Philox call each)
  for (int64_t g = tid; 4 * g < V; g += kSmT) {
    float z[4];
    bool in[4], any = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = 4 * g + e;
      z[e] = i < V ? val<T>(zrow, i) : -INFINITY;
      in[e] = z[e] >= tau && z[e] > -INFINITY;
      any |= in[e];
    }
    if (!any) continue;
    uint32_t c[4] = {uint32_t(g), uint32_t(rk), uint32_t(rk >> 32), a.offset};
    philox4x32_10(c, k0, k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!in[e]) continue;
      const double u = (double(c[e]) + 0.5) * 0x1p-32;
      const double s = double(z[e]) / T64 - log(-log(u));
      if (better(s, 4 * g + e, best, best_i)) {
        best = s;
        best_i = 4 * g + e;
      }
    }
  }
  // block argmax: a fixed butterfly in each wave, then the waves in order
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const double s2 = __shfl_xor(best, off, kWave);
    const int64_t i2 = __shfl_xor(best_i, off, kWave);
    if (better(s2, i2, best, best_i)) {
      best = s2;
      best_i = i2;
    }
  }
  if (lane == 0) {
    ss[wid] = best;
    si[wid] = best_i;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSmT / kWave; ++w)
      if (better(ss[w], si[w], best, best_i)) {
        best = ss[w];
        best_i = si[w];
      }
    a.samples[row] = best_i == INT64_MAX ? -1 : best_i;
  }
}

__global__ void fill_i64(int64_t* p, int64_t n, int64_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_sample_rows(const SampleArgs& a, int dtype, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_rows));
  if (dtype == 0)
    hipLaunchKernelGGL(sample_rows<float>, grid, dim3(kSmT), 0, stream, a);
  else
    hipLaunchKernelGGL(sample_rows<uint16_t>, grid, dim3(kSmT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fill_i64(int64_t* p, int64_t n, int64_t v, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(fill_i64, dim3(unsigned(blocks)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace rlk
