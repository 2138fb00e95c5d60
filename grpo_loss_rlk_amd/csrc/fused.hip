// Fused LM head: token log-probability and entropy under softmax(h W^T / T)
// without materialising the [N, V] logits (prime-rl v0.10.0 release notes,
// "1. Trainer Performance": the loss is chunked torchtitan-style).
//
// Forward at top-p = 1, two launches:
//  1. fwd_tile_stats: one block per (256-vocab x 256-token) tile; z = W h^T
//     in fp32 on bf16 MFMA (mfma_gemm.h). The epilogue folds the tile's 256
//     logits of each token into a partial (max z, sum 2^x, sum 2^x x) with
//     x = (z - max) log2(e)/T, and the block whose vocabulary slice holds a
//     token's target writes that target logit.
//  2. fwd_merge: per token, the ceil(V/256) partials are merged in fp64 in a
//     fixed order that depends on V only, so results do not depend on the
//     number of tokens or their order (the Qwen3-8B VIME consistency page,
//     "Canonical topology strategy", combines vocabulary shards in one fixed
//     order).
//
// Forward at top-p < 1 or with top-k (the cut needs the whole row): per
// block of kTopPRowBlock tokens, fwd_logits_tile writes the block's fp32
// logits z = h W^T to a workspace scratch [rows, Vs] and the logits-in row
// kernel (max, nucleus by value histogram, truncated statistics) cuts each
// row at the tempered top-p threshold.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "fused_kernels.h"
#include "kernels.h"
#include "mfma_gemm.h"

namespace rlk {

namespace {

using gemm::f32x16;
constexpr int kBM = gemm::kTile;   // vocabulary rows per block
constexpr int kBN = gemm::kTile;   // tokens per block
constexpr int kT = gemm::kThreads;
constexpr float kLn2 = 0.6931471805599453f;

// Merge of softmax partials (max m in z units, A = sum 2^x, B = sum 2^x x with
// x in log2 units of the scaled logit). c2 = log2(e)/T.
struct Part {
  float m, A, B;
};

RLK_DEV Part merge_part(Part p, Part q, float c2) {
  if (p.m != p.m || q.m != q.m) return Part{p.m + q.m, 0.f, 0.f};   // a non-finite logit: NaN
  if (q.m == -INFINITY) return p;   // an empty partial (no valid vocabulary rows)
  if (p.m == -INFINITY) return q;
  const float m = fmaxf(p.m, q.m);
  const float dp = (p.m - m) * c2, dq = (q.m - m) * c2;
  const float sp = exp2f(dp), sq = exp2f(dq);
  Part r;
  r.m = m;
  r.A = p.A * sp + q.A * sq;
  r.B = sp * (p.B + dp * p.A) + sq * (q.B + dq * q.A);
  return r;
}

// This lane's 64 logits of token column j folded into (max, sum 2^x, sum 2^x x).
// kFull: every vocabulary row of the tile exists; else rows from `rem` on
// (relative to this lane's first row) are past the vocabulary and are left
// out. `rem` passes through an empty asm per column and per pass, so that the
// 64 comparisons are made afresh each time rather than shared and kept live:
// their masks would not fit the scalar registers. A NaN or
// infinite logit makes the partial's max NaN, which every merge propagates;
// it is detected by a sum of z * 0, which stays 0 for finite z. That sum
// includes rows past the vocabulary: the GEMM loaded them as copies of the
// last vocabulary row, which lies in the same tile, so they are non-finite
// only where a real logit of this token is, and the token's merged result is
// NaN either way.
template <bool kFull>
RLK_DEV Part fold_lane(const f32x16 (&acc)[4][4], int j, int rem, float c2) {
  float mx = -INFINITY, chk = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float z = acc[i][j][r];
      chk = fmaf(z, 0.f, chk);
      if (kFull || 32 * i + 8 * (r >> 2) + (r & 3) < rem) mx = fmaxf(mx, z);
    }
  if (!(chk == 0.f)) return Part{__builtin_nanf(""), 0.f, 0.f};
  float A = 0.f, B = 0.f;
  if (mx > -INFINITY) {
    if (!kFull) asm volatile("" : "+v"(rem));   // fresh comparisons, as above
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // x <= 0; below 2^-126 a term is far under the sum's resolution,
        // whatever the denormal handling of the hardware exp2. The clamp
        // changes no term (exp2 of anything below -150 is 0 in fp32) and
        // gives rows past the vocabulary a zero term.
        float x = fmaxf((acc[i][j][r] - mx) * c2, -1024.f);
        if (!kFull && !(32 * i + 8 * (r >> 2) + (r & 3) < rem)) x = -1024.f;
        const float e = __builtin_amdgcn_exp2f(x);
        A += e;
        B = fmaf(e, x, B);
      }
  }
  return Part{mx, A, B};
}

// Epilogue of a 256 x 256 tile: per token, fold this tile's logits into a
// partial and write the target logit; `xch` is >= 3 KB of free LDS.
RLK_DEV void tile_epilogue(const FusedFwdArgs& a, f32x16 (&acc)[4][4], int64_t v0, int64_t n0,
                           int vt, float* xch) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int frow = lane & 31, fgrp = lane >> 5;
  // accumulator acc[i][j][r] holds vocab row 128*wm + 32*i + 8*(r/4) + 4*fgrp + r%4
  // and token 128*wn + 32*j + frow of the tile.
  const float c2 = a.c2;
  const int64_t vbase = v0 + 128 * wm;
  const bool full = v0 + kBM <= a.V;
  const int64_t rem64 = a.V - vbase - 4 * fgrp;
  const int rem = int(rem64 < 256 ? rem64 : 256);
  // the four token columns' targets, loaded together so that one memory
  // latency is exposed instead of a chain of four
  int64_t yv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + 128 * wn + 32 * j + frow;
    yv[j] = n < a.N ? a.targets[n] : -1;
  }
  Part mine[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int remj = rem;
    asm volatile("" : "+v"(remj));
    const Part p = full ? fold_lane<true>(acc, j, remj, c2) : fold_lane<false>(acc, j, remj, c2);
    Part q;
    q.m = __shfl_xor(p.m, 32, 64);
    q.A = __shfl_xor(p.A, 32, 64);
    q.B = __shfl_xor(p.B, 32, 64);
    // lanes l and l^32 hold the same token: merge the lower half first
    mine[j] = fgrp == 0 ? merge_part(p, q, c2) : merge_part(q, p, c2);

    // target logit: the lane holding vocab row y of this token writes it
    const int64_t n = n0 + 128 * wn + 32 * j + frow;
    const int64_t y = yv[j];
    const int64_t rel = y - vbase;
    const bool hit = rel >= 0 && rel < 128 && ((rel >> 2) & 1) == fgrp;
    if (__any(hit)) {
      // element (i, r) = (rel / 32, 4 (rel % 32 / 8) + rel % 4), picked by a
      // select tree over the 6 bits of 16 i + r (6 masks, not 64)
      const int ww = int(rel & 31);
      const int idx = (int(rel >> 5) << 4) | ((ww >> 3) << 2) | (ww & 3);
      float t[64];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) t[16 * i + r] = acc[i][j][r];
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const bool bit = (idx >> b) & 1;
#pragma unroll
        for (int k = 0; k < (32 >> b); ++k) t[k] = bit ? t[2 * k + 1] : t[2 * k];
      }
      if (hit) a.zy[n] = t[0];
    }
  }

  // ---- combine the two vocab halves (wm = 0 then 1) and write partials ----
  if (wm == 1 && fgrp == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 32 * j + frow;
      xch[(wn * 128 + t) * 3 + 0] = mine[j].m;
      xch[(wn * 128 + t) * 3 + 1] = mine[j].A;
      xch[(wn * 128 + t) * 3 + 2] = mine[j].B;
    }
  }
  __syncthreads();
  if (wm == 0 && fgrp == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 32 * j + frow;
      const int64_t n = n0 + 128 * wn + t;
      Part o{xch[(wn * 128 + t) * 3 + 0], xch[(wn * 128 + t) * 3 + 1],
             xch[(wn * 128 + t) * 3 + 2]};
      const Part r = merge_part(mine[j], o, c2);
      if (n < a.N) a.part[int64_t(vt) * a.N + n] = make_float4(r.m, r.A, r.B, 0.f);
    }
  }
}

__global__ __launch_bounds__(kT) void fwd_tile_stats(FusedFwdArgs a) {
  __shared__ gemm::Smem smem;
  const int nvt = int((a.V + kBM - 1) / kBM), nnt = int((a.N + kBN - 1) / kBN);
  int vt, nt;
  gemm::tile_of_block(nvt, nnt, vt, nt);
  const int64_t v0 = int64_t(vt) * kBM, n0 = int64_t(nt) * kBN;
  f32x16 acc[4][4];
  gemm::gemm_nt_tile(acc, smem, a.w, v0, a.V, a.ws, a.h, n0, a.N, a.hs, a.H);
  tile_epilogue(a, acc, v0, n0, vt, reinterpret_cast<float*>(&smem[0][0][0]));
}

// Logits of a row block: A = W (vocabulary), B = h (tokens), the
// orientation (and tile order) of fwd_tile_stats, so that W is streamed once
// per row block in bands of 32 vocabulary tiles. A lane's accumulators acc[i][j][4 s + e],
// e = 0..3, are 4 consecutive ids of one token, so each goes to the scratch
// row as one 16-byte store straight from registers (lanes l and l + 32 write
// the two halves of 32 contiguous bytes; the 4 values of s complete a
// token's 128-byte line). Per token: the max logit over the tile (as an order
// key, merged with atomicMax, which is order-free) and whether a non-finite
// logit appeared (a sum of z * 0 is NaN), so that the row kernel can skip its
// max pass; one atomic per token and wave.
template <bool kFullV>
RLK_DEV void logits_epilogue(f32x16 (&acc)[4][4], int64_t v0, int64_t n0, int64_t V,
                             int64_t rows, float* z, int64_t zs, uint32_t* zmax_key,
                             uint32_t* zbad) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = int(threadIdx.x) & 63;
  const int64_t vb = v0 + gemm::acc_a_row(0, 0);   // this lane's first id
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + gemm::acc_b_row(j);
    // a fresh copy per column: the 64 id comparisons are then made per column
    // rather than shared and kept live (their masks would not fit the scalar
    // registers)
    int64_t vrem = V - vb;
    if (!kFullV) asm volatile("" : "+v"(vrem));
    float mx = -INFINITY, chk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int k0 = 32 * i + 8 * s4;   // ids vb + k0 .. + 3
        const f32x4 v = {acc[i][j][4 * s4], acc[i][j][4 * s4 + 1], acc[i][j][4 * s4 + 2],
                         acc[i][j][4 * s4 + 3]};
        // zs is a multiple of 4, so a chunk that starts inside the row ends inside it
        if (n < rows && vb + k0 < zs) *reinterpret_cast<f32x4*>(z + n * zs + vb + k0) = v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          chk = fmaf(v[e], 0.f, chk);   // rows past V are copies of row V - 1
          if (kFullV || k0 + e < vrem) mx = fmaxf(mx, v[e]);
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    chk = chk + __shfl_xor(chk, 32, 64);
    if (lane < 32 && n < rows) {
      if (mx > -INFINITY) atomicMax(&zmax_key[n], f32_key(mx));
      if (!(chk == 0.f)) atomicOr(&zbad[n], 1u);
    }
  }
}

__global__ __launch_bounds__(kT) void fwd_logits_tile(FusedFwdArgs a, int64_t r0, int64_t rows,
                                                      float* z, int64_t zs, uint32_t* zmax_key,
                                                      uint32_t* zbad) {
  __shared__ gemm::Smem smem;
  const int nvt = int((a.V + kBM - 1) / kBM), nnt = int((rows + kBN - 1) / kBN);
  int vt, nt;
  gemm::tile_of_block(nvt, nnt, vt, nt);
  const int64_t v0 = int64_t(vt) * kBM, n0 = int64_t(nt) * kBN;
  f32x16 acc[4][4];
  gemm::gemm_nt_tile(acc, smem, a.w, v0, a.V, a.ws, a.h + r0 * a.hs, n0, rows, a.hs, a.H);
  if (v0 + kBM <= a.V)
    logits_epilogue<true>(acc, v0, n0, a.V, rows, z, zs, zmax_key, zbad);
  else
    logits_epilogue<false>(acc, v0, n0, a.V, rows, z, zs, zmax_key, zbad);
}

__global__ void clear_u32(uint32_t* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Merge of the per-tile partials of each token, in fp64: the row max m is
// the max of the tile maxima (exact), then A = sum_t A_t 2^{(m_t - m) c2} and
// B = sum_t 2^{(m_t - m) c2} (B_t + (m_t - m) c2 A_t). A block holds 32 tokens
// x 8 slices; slice s sums tiles s, s + 8, s + 16, ... in increasing order and
// the slices are added in slice order, so the summation order depends on the
// number of vocabulary tiles only.
constexpr int kMergeTok = 32, kMergeSlices = 8;

__global__ __launch_bounds__(kMergeTok * kMergeSlices) void fwd_merge(FusedFwdArgs a, int nvt) {
  __shared__ double sh[3][kMergeSlices][kMergeTok];
  const int tok = threadIdx.x & (kMergeTok - 1), sl = threadIdx.x / kMergeTok;
  const int64_t n = int64_t(blockIdx.x) * kMergeTok + tok;
  const bool live = n < a.N;
  const double c2 = double(a.c2);

  float mx = -INFINITY;
  if (live)
    for (int vt = sl; vt < nvt; vt += kMergeSlices) {
      const float px = a.part[int64_t(vt) * a.N + n].x;
      mx = (px != px || mx != mx) ? __builtin_nanf("") : fmaxf(mx, px);   // NaN: non-finite logit
    }
  sh[0][sl][tok] = double(mx);
  __syncthreads();
  double m = -INFINITY;
  bool bad = false;   // a tile saw a NaN or infinite logit
  for (int k = 0; k < kMergeSlices; ++k) {
    m = sh[0][k][tok] > m ? sh[0][k][tok] : m;
    bad |= sh[0][k][tok] != sh[0][k][tok];
  }
  __syncthreads();

  double A = 0.0, B = 0.0;   // B in log2 units
  if (live && !bad && m > -INFINITY)
    for (int vt = sl; vt < nvt; vt += kMergeSlices) {
      const float4 p = a.part[int64_t(vt) * a.N + n];
      if (!(p.x > -INFINITY)) continue;   // a tile with no valid vocabulary row
      const double d = (double(p.x) - m) * c2;
      const double sc = exp2(d);
      A += double(p.y) * sc;
      B += sc * (double(p.z) + d * double(p.y));
    }
  sh[1][sl][tok] = A;
  sh[2][sl][tok] = B;
  __syncthreads();
  if (sl != 0 || !live) return;
  A = 0.0;
  B = 0.0;
  for (int k = 0; k < kMergeSlices; ++k) {
    A += sh[1][k][tok];
    B += sh[2][k][tok];
  }
  const double invT = c2 * double(kLn2);    // 1/T
  const double lnA = log(A);
  const double Ed = double(kLn2) * B / A;   // E_q[(z - m)/T] in nats
  const double H = lnA - Ed;
  const int64_t y = a.targets[n];
  uint8_t flags = 0;
  float lp;
  if (y < 0 || y >= a.V) {
    flags |= 2;
    lp = __builtin_nanf("");
  } else {
    lp = float((double(a.zy[n]) - m) * invT - lnA);
  }
  const float nan = __builtin_nanf("");
  if (bad || !(m > -INFINITY)) flags |= 4;   // a NaN / infinite logit, or no finite one
  a.logprob[n] = (flags & 4) ? nan : lp;
  a.entropy[n] = (flags & 4) ? nan : float(H);
  if (a.saved) {
    a.saved[4 * n + 0] = (flags & 4) ? nan : float(m * invT + lnA);   // log Z of z/T
    a.saved[4 * n + 1] = (flags & 4) ? nan : float(m * invT + Ed);    // E_q[z/T]
    a.saved[4 * n + 2] = -INFINITY;              // no cut at top-p = 1
    a.saved[4 * n + 3] = (flags & 6) ? 0.f : 1.f;  // the lp term is live (target in range)
  }
  if (a.nsize) a.nsize[n] = int32_t(a.V);
  if (a.flags) a.flags[n] = flags;
}

}  // namespace

namespace {

int64_t logits_ld(int64_t V) { return (V + 63) / 64 * 64; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t fused_fwd_workspace(int64_t N, int64_t H, int64_t V, float top_p, int32_t top_k) {
  (void)H;
  if (top_p < 1.f || top_k > 0) {
    const int64_t R = N < kTopPRowBlock ? N : kTopPRowBlock;
    return align256(size_t(R) * size_t(logits_ld(V)) * 4) + align256(size_t(N) * 4) +
           2 * align256(size_t(R) * 4) + logits_rows_workspace(R, V, 0);
  }
  const int64_t nvt = (V + kBM - 1) / kBM;
  return size_t(nvt * N) * 16 + size_t(N) * 4 + 512;
}

hipError_t launch_fused_fwd(FusedFwdArgs a, void* workspace, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  char* ws = reinterpret_cast<char*>(workspace);
  if (a.top_p < 1.f || a.top_k > 0) {
    const int64_t R = a.N < kTopPRowBlock ? a.N : kTopPRowBlock, zs = logits_ld(a.V);
    float* z = reinterpret_cast<float*>(ws);
    size_t off = align256(size_t(R) * size_t(zs) * 4);
    float* lp_full = reinterpret_cast<float*>(ws + off);
    off += align256(size_t(a.N) * 4);
    uint32_t* zmax_key = reinterpret_cast<uint32_t*>(ws + off);
    off += align256(size_t(R) * 4);
    uint32_t* zbad = reinterpret_cast<uint32_t*>(ws + off);
    off += align256(size_t(R) * 4);
    void* rows_ws = ws + off;
    // the row kernel clears both per-row arrays after reading them
    hipLaunchKernelGGL(clear_u32, dim3(unsigned((2 * align256(size_t(R) * 4) / 4 + 255) / 256)),
                       dim3(256), 0, stream, zmax_key, int64_t(2 * align256(size_t(R) * 4) / 4));
    for (int64_t r0 = 0; r0 < a.N; r0 += R) {
      const int64_t rows = a.N - r0 < R ? a.N - r0 : R;
      const int64_t nnt = (rows + kBN - 1) / kBN, nvt = (a.V + kBM - 1) / kBM;
      hipLaunchKernelGGL(fwd_logits_tile, dim3(unsigned(nnt * nvt)), dim3(kT), 0, stream, a, r0,
                         rows, z, zs, zmax_key, zbad);
      RowArgs ra{};
      ra.logits = z;
      ra.n_rows = rows;
      ra.vocab = a.V;
      ra.row_stride = zs;
      ra.targets = a.targets + r0;
      ra.temperature = a.temperature;
      ra.top_p = a.top_p;
      ra.top_k = a.top_k;
      ra.lp_full = lp_full + r0;
      ra.lp_trunc = a.logprob + r0;
      ra.ent_trunc = a.entropy + r0;
      ra.nsize = a.nsize ? a.nsize + r0 : nullptr;
      ra.flags = a.flags ? a.flags + r0 : nullptr;
      ra.saved4 = a.saved ? a.saved + 4 * r0 : nullptr;
      ra.zmax_key = zmax_key;
      ra.zbad = zbad;
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      e = launch_logits_rows(ra, 0, rows_ws, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int64_t nvt = (a.V + kBM - 1) / kBM, nnt = (a.N + kBN - 1) / kBN;
  a.part = reinterpret_cast<float4*>(ws);
  a.zy = reinterpret_cast<float*>(ws + (size_t(nvt * a.N) * 16 + 255) / 256 * 256);
  hipLaunchKernelGGL(fwd_tile_stats, dim3(unsigned(nvt * nnt)), dim3(kT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_merge, dim3(unsigned((a.N + kMergeTok - 1) / kMergeTok)),
                     dim3(kMergeTok * kMergeSlices), 0, stream, a, int(nvt));
  return hipGetLastError();
}

}  // namespace rlk
