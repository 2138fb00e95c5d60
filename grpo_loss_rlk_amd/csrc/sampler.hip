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
constexpr uint8_t kOutside = 1, kBadTarget = 2, kNonFinite = 4, kBadParam = 16;

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

// The drawn token y scored as the logits-in kernel scores a target (the same
// token_logprob from the nucleus pass's row max and log Z_S): the nucleus
// pass's flags without its placeholder target's bits, and for y < 0 (no
// draw) the out-of-range bit and a NaN logprob.
template <typename T>
RLK_DEV void score_draw(const SampleArgs& a, int64_t row, const T* zrow, int64_t y) {
  const uint8_t f = a.nflags[row] & uint8_t(~(kOutside | kBadTarget));
  float lp = __builtin_nanf("");
  const float Tv = a.t_row ? a.t_row[row] : a.temperature;
  if (y >= 0)
    lp = token_logprob(val<T>(zrow, y), a.score_stats[2 * row], 1.0 / double(Tv),
                       a.score_stats[2 * row + 1]);
  if (a.logprob) a.logprob[row] = lp;
  if (a.flags) a.flags[row] = y >= 0 ? f : uint8_t(f | kBadTarget);
}

// (score, id) order: higher score first, then the lower id
RLK_DEV bool better(double s, int64_t i, double s2, int64_t i2) {
  return s > s2 || (s == s2 && i < i2);
}

constexpr int kAhead = 8;   // 16-byte vectors in flight per thread

// One row per block. Each round, a wave reads 64 consecutive 16-byte vectors
// (one per lane; kAhead rounds in flight) and appends the ids of its nucleus
// members (logit >= tau) to its own list in LDS (a wave prefix sum places
// each lane's entries). The list is scored densely across the wave's lanes
// (so the Philox and fp64 work is not spread thin over diverged lanes; the
// logit is read again, from cache) only when the next round might overflow
// it and at the end of the row, so a sparse nucleus costs a few scoring
// passes per row rather than one per round. The waves never wait for one
// another until the final argmax: a wave's LDS accesses are performed in
// order, so its list needs no block barrier. The draw is an argmax under a total order (higher
// score, then lower id), so neither the order of a list nor the split of the
// row over waves changes it.
template <typename T, bool kVec>
__global__ __launch_bounds__(kSmT) void sample_rows(SampleArgs a) {
  constexpr int kEV = 16 / int(sizeof(T));   // values per 16-byte vector (8 bf16, 4 fp32)
  __shared__ double ss[kSmT / kWave];
  __shared__ int64_t si[kSmT / kWave];
  constexpr int kCap = 2 * kWave * kEV;   // a wave's list: two rounds' worth of ids
  __shared__ int32_t list_i[kSmT / kWave][kCap];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t row = blockIdx.x;
  const T* zrow = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  if (a.nflags[row] & (kNonFinite | kBadParam)) {
    if (tid == 0) {
      a.samples[row] = -1;
      score_draw<T>(a, row, zrow, -1);
    }
    return;
  }
  const int64_t V = a.vocab;
  const float tau = a.thresh[row];
  const double T64 = double(a.t_row ? a.t_row[row] : a.temperature);
  const uint64_t rk = a.row_keys ? uint64_t(a.row_keys[row]) : uint64_t(row);
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  double best = -INFINITY;
  int64_t best_i = INT64_MAX;
  int32_t* lst = list_i[wid];

  int listed = 0;   // entries in this wave's list (wave-uniform)

  // score this wave's listed ids densely across its lanes and empty the list
  auto score = [&]() __attribute__((always_inline)) {
    // the wave's list writes before its reads (compiler order; the hardware
    // performs one wave's LDS accesses in order)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int c = lane; c < listed; c += kWave) {
      const int64_t i = lst[c];
      uint32_t w[4] = {uint32_t(i >> 2), uint32_t(rk), uint32_t(rk >> 32), a.offset};
      philox4x32_10(w, k0, k1);
      const uint32_t word = (i & 3) == 0 ? w[0] : (i & 3) == 1 ? w[1] : (i & 3) == 2 ? w[2] : w[3];
      const double u = (double(word) + 0.5) * 0x1p-32;
      const double s = double(val<T>(zrow, i)) / T64 - log(-log(u));
      if (better(s, i, best, best_i)) {
        best = s;
        best_i = i;
      }
    }
    // the reads before later writes
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    listed = 0;
  };
  // append this lane's ids i0 .. i0 + kEV - 1 that are in the nucleus to the
  // wave's list, scoring the list first if this round might not fit; the
  // whole wave calls this together
  auto offer = [&](int64_t i0, const float (&z)[kEV]) __attribute__((always_inline)) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kEV; ++e)
      if (i0 + e < V && z[e] >= tau && z[e] > -INFINITY) m |= 1u << e;
    const int n = __popc(m);
    const int incl = wave_scan_incl(n);
    const int total = __shfl(incl, kWave - 1, kWave);
    if (total == 0) return;
    if (listed + total > kCap) score();
    int base = listed + incl - n;
    while (m) {
      const int e = __ffs(m) - 1;
      m &= m - 1;
      lst[base] = int32_t(i0 + e);
      ++base;
    }
    listed += total;
  };
  auto unpack = [&](const uint4& q, float (&z)[kEV]) __attribute__((always_inline)) {
    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
    if (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[2 * e] = __uint_as_float(wv[e] << 16);
        z[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = __uint_as_float(wv[e]);
    }
  };

  if (kVec) {
    const uint4* v4 = reinterpret_cast<const uint4*>(zrow);
    const int64_t nvec = (V + kEV - 1) / kEV;   // the last vector may run past V (row padding)
    const int64_t full = V / kEV;
    // kAhead vectors per thread in flight: round r consumes slot r % kAhead
    // and refills it with round r + kAhead's vector
    uint4 q[kAhead];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) {
      const int64_t j = int64_t(s) * kSmT + tid;
      q[s] = j < full ? v4[j] : make_uint4(0, 0, 0, 0);
    }
    for (int64_t r0 = 0; r0 < nvec; r0 += int64_t(kSmT) * kAhead) {
#pragma unroll
      for (int s = 0; s < kAhead; ++s) {
        const int64_t rs = r0 + int64_t(s) * kSmT;
        if (rs >= nvec) break;   // uniform
        const int64_t j = rs + tid;
        float z[kEV];
        unpack(q[s], z);
        const int64_t jn = j + int64_t(kSmT) * kAhead;
        q[s] = jn < full ? v4[jn] : make_uint4(0, 0, 0, 0);
        if (j >= full) {   // the partial last vector, element by element
#pragma unroll
          for (int e = 0; e < kEV; ++e) {
            const int64_t i = j * kEV + e;
            z[e] = (j < nvec && i < V) ? val<T>(zrow, i) : -INFINITY;
          }
        }
        offer(j * kEV, z);
      }
    }
  } else {
    for (int64_t r0 = 0; r0 < V; r0 += int64_t(kSmT) * kEV) {
      float z[kEV];
#pragma unroll
      for (int e = 0; e < kEV; ++e) {
        const int64_t i = r0 + int64_t(tid) * kEV + e;
        z[e] = i < V ? val<T>(zrow, i) : -INFINITY;
      }
      offer(r0 + int64_t(tid) * kEV, z);
    }
  }
  if (listed > 0) score();
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
    const int64_t y = best_i == INT64_MAX ? -1 : best_i;
    a.samples[row] = y;
    score_draw<T>(a, row, zrow, y);
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
  const size_t esz = dtype == 0 ? 4 : 2;
  const bool vec = reinterpret_cast<uintptr_t>(a.logits) % 16 == 0 && (a.row_stride * esz) % 16 == 0;
  if (dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((sample_rows<float, true>), grid, dim3(kSmT), 0, stream, a);
    else
      hipLaunchKernelGGL((sample_rows<float, false>), grid, dim3(kSmT), 0, stream, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((sample_rows<uint16_t, true>), grid, dim3(kSmT), 0, stream, a);
    else
      hipLaunchKernelGGL((sample_rows<uint16_t, false>), grid, dim3(kSmT), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fill_i64(int64_t* p, int64_t n, int64_t v, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(fill_i64, dim3(unsigned(blocks)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace rlk
