// Fused LM head, backward by chunk recompute (prime-rl v0.10.0 release
// notes, "1. Trainer Performance": the chunked loss recomputes the logits of
// a vocabulary chunk instead of storing them).
//
// With z = h W^T, x = z/T, q = exp(x - log Z) and the forward's saved
// statistics (log Z and E_q[x] per token), the gradient with respect to the
// logits is
//   G[n,i] = (1/T) [ g_lp (delta_{i,y} - q_i) - g_H q_i (x_i - E_q[x]) ],
// and grad_hidden = G W, grad_weight = G^T h. Per vocabulary chunk c of
// kBwdChunk rows, in a fixed chunk order:
//   1. bwd_g_tile:  S_c = W_c h^T on MFMA; the epilogue forms G_c in bf16 and
//      stores it twice, as [N, C] (token rows) and as [C, N] (vocabulary rows),
//      zero-padded, so that both products below read K-contiguous operands.
//   2. bwd_dh_tile: dh (+)= G_c W_c, with W^T (transposed once per call) as the
//      K-contiguous operand; fp32 partial sums across chunks, bf16 at the end.
//   3. bwd_dw_tile: dW_c = G_c^T h, with h^T (transposed once per call).
// All three are the tile GEMM of mfma_gemm.h.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "fused_kernels.h"
#include "mfma_gemm.h"

namespace rlk {

namespace {

using gemm::f32x16;
constexpr int kTile = gemm::kTile;
constexpr int kT = gemm::kThreads;
constexpr float kLog2e = 1.4426950408889634f;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

RLK_DEV uint16_t to_bf16(float f) {   // round to nearest even; NaN stays NaN
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// dst[c, r] = src[r, c] for c < cols, r < rows; zero for rows <= r < dst_ld.
// One 64 x 64 block per workgroup: grid (dst_ld / 64, cols / 64).
__global__ __launch_bounds__(256) void transpose_pad(const uint16_t* src, int64_t rows,
                                                     int64_t src_ld, uint16_t* dst,
                                                     int64_t dst_ld) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = int64_t(blockIdx.x) * 64, c0 = int64_t(blockIdx.y) * 64;
  const int tid = threadIdx.x, row = tid >> 2, seg = tid & 3;
  {
    const int64_t r = r0 + row;
    uint4 v[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    if (r < rows) {
      const uint4* p = reinterpret_cast<const uint4*>(src + r * src_ld + c0 + seg * 16);
      v[0] = p[0];
      v[1] = p[1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t x = k < 4 ? (&v[0].x)[k] : (&v[1].x)[k - 4];
      t[row][seg * 16 + 2 * k] = uint16_t(x);
      t[row][seg * 16 + 2 * k + 1] = uint16_t(x >> 16);
    }
  }
  __syncthreads();
  {
    const int c = row;   // output row (input column) c0 + c, output columns r0 + seg*16 ..
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = uint32_t(t[seg * 16 + 2 * k][c]) | (uint32_t(t[seg * 16 + 2 * k + 1][c]) << 16);
    uint4* q = reinterpret_cast<uint4*>(dst + (c0 + c) * dst_ld + r0 + seg * 16);
    q[0] = make_uint4(w[0], w[1], w[2], w[3]);
    q[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

__global__ __launch_bounds__(256) void fill_f32(float* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = 0.f;
}

// Row strides of the workspace matrices are 64 elements (128 bytes) past a
// multiple of 64, so never a multiple of a large power of two: a GEMM stage
// reads 256 rows at one k offset, and at a stride of 64 KB (a 32768-row chunk)
// those rows' lines crowd onto a few memory channels (the dh product ran 4-6 %
// slower at that stride than at 64 KB + 128 bytes).
constexpr int64_t kLdPad = 64;
// rows and vocabularies below 2^23 (checked at the boundary) keep every
// padded stride within the tile GEMM's limit
static_assert((int64_t(1) << 23) + kLdPad <= gemm::kMaxLd, "padded strides fit the copy offsets");

struct ChunkArgs {
  int64_t c0, csz, cpad;   // chunk start, rows, rows padded to a multiple of 64
  int64_t cap;             // row stride of g_nc (chunk capacity + kLdPad)
  int64_t npad;            // tokens padded to a multiple of 64 (the dW product's K)
  int64_t nld;             // row stride of g_cn and h^T (npad + kLdPad)
  uint16_t* g_nc;          // bf16 [N, cap]    G_c, token rows
  uint16_t* g_cn;          // bf16 [cap, nld]  G_c^T, vocabulary rows
  const uint16_t* wt;      // bf16 [H, vld]    W^T
  int64_t vld;             // row stride of W^T (V padded to 64, + kLdPad)
  const uint16_t* ht;      // bf16 [H, nld]    h^T
  float* dh_acc;           // fp32 [N, H] partial sums over chunks (several chunks only)
};

// G of one S_c tile from the accumulators: each element to bf16, into the
// LDS tile tg [vocabulary][token] and, four vocabulary rows at a time, to the
// token-row copy g_nc. kFullV: all 256 vocabulary rows of the tile are in the
// chunk. A token past N gets lse = +huge, so q = 0 and G = +0 without a mask.
// The nucleus is the forward's: logits >= tau (saved slot 2, -inf at top-p =
// 1) are kept, the recomputed logits being the forward's fp32 sums over the
// same k order; the lp term counts only where the forward found the target
// kept (saved slot 3).
template <bool kFullV>
RLK_DEV void g_epilogue(const FusedBwdArgs& a, const ChunkArgs& c, const f32x16 (&acc)[4][4],
                        int64_t v0, int64_t n0, uint16_t* tg) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int rbase = gemm::acc_a_row(0, 0);   // 128 wm + 4 (lane / 32): this lane's first row
  const float inv_t = a.inv_t, c1 = inv_t * kLog2e;
  const int vrem = int(c.csz - v0 < 2 * kTile ? c.csz - v0 : 2 * kTile) - rbase;
  // the four token columns' inputs, loaded together (a token past N reads
  // row N - 1 and is then ignored) so that one memory latency is exposed
  // instead of a chain of dependent ones per column
  float sv[4][4], ghv[4], glv[4];
  int64_t yv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + gemm::acc_b_row(j);
    const int64_t nc = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[j][k] = a.saved[4 * nc + k];
    ghv[j] = a.g_H ? a.g_H[nc] : 0.f;
    glv[j] = a.g_lp ? a.g_lp[nc] : 0.f;
    yv[j] = a.targets[nc];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = gemm::acc_b_row(j);
    const int64_t n = n0 + nl;
    // a fresh copy per column: the 64 row comparisons below are then made per
    // column rather than shared and kept live (their masks would not fit the
    // scalar registers)
    int vremj = vrem;
    if (!kFullV) asm volatile("" : "+v"(vremj));
    float lse2 = 1e30f, eq = 0.f, glp = 0.f, gh = 0.f, tau = -INFINITY;
    int ty = -1;   // target row relative to this lane's first row (-1: none here)
    if (n < a.N) {
      lse2 = sv[j][0] * kLog2e;
      eq = sv[j][1];
      tau = sv[j][2];
      gh = ghv[j];
      const int64_t y = yv[j];
      // a row whose target is out of range or outside the nucleus keeps only
      // its entropy term
      if (y >= 0 && y < a.V && sv[j][3] != 0.f) {
        glp = glv[j];
        const int64_t rel = y - c.c0 - v0 - rbase;
        ty = rel >= 0 && rel < kTile ? int(rel) : -1;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k0 = 32 * i + 8 * s;   // rows rbase + k0 .. + 3
        float g4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = acc[i][j][4 * s + e];
          const float q = !(z < tau) ? __builtin_amdgcn_exp2f(fmaf(z, c1, -lse2)) : 0.f;  // NaN stays
          float g = fmaf(-q, fmaf(gh, fmaf(z, inv_t, -eq), glp), 0.f);   // +0 when q = 0
          if (k0 + e == ty) g += glp;
          g *= inv_t;
          if (!kFullV && k0 + e >= vremj) g = 0.f;
          g4[e] = g;
        }
        const bf16x2 lo = {(__bf16)g4[0], (__bf16)g4[1]};
        const bf16x2 hi = {(__bf16)g4[2], (__bf16)g4[3]};
        const uint32_t plo = __builtin_bit_cast(uint32_t, lo), phi = __builtin_bit_cast(uint32_t, hi);
        uint16_t* t = tg + (rbase + k0) * kTile + nl;
        t[0] = uint16_t(plo);
        t[kTile] = uint16_t(plo >> 16);
        t[2 * kTile] = uint16_t(phi);
        t[3 * kTile] = uint16_t(phi >> 16);
        const int64_t vb = v0 + rbase + k0;
        if (vb < c.cpad && n < a.N)
          *reinterpret_cast<uint2*>(c.g_nc + n * c.cap + vb) = make_uint2(plo, phi);
      }
  }
}

// S_c tile (vocabulary rows of the chunk x tokens) and its G epilogue.
__global__ __launch_bounds__(kT) void bwd_g_tile(FusedBwdArgs a, ChunkArgs c) {
  __shared__ gemm::Smem smem;
  const int nvt = int((c.csz + kTile - 1) / kTile), nnt = int((a.N + kTile - 1) / kTile);
  int vt, nt;
  gemm::tile_of_block(nvt, nnt, vt, nt);
  const int64_t v0 = int64_t(vt) * kTile, n0 = int64_t(nt) * kTile;
  f32x16 acc[4][4];
  gemm::gemm_nt_tile(acc, smem, a.w + c.c0 * a.ws, v0, c.csz, a.ws, a.h, n0, a.N, a.hs, a.H);

  // G of the tile, [vocabulary][token] in LDS, for the row-contiguous G^T stores
  uint16_t* tg = reinterpret_cast<uint16_t*>(&smem[0][0][0]);
  static_assert(sizeof(gemm::Smem) >= kTile * kTile * 2, "the G tile fits the GEMM's LDS");
  if (v0 + kTile <= c.csz)
    g_epilogue<true>(a, c, acc, v0, n0, tg);
  else
    g_epilogue<false>(a, c, acc, v0, n0, tg);
  __syncthreads();
  // G^T rows: 256 tokens (512 bytes) per vocabulary row, 16 bytes per thread
  constexpr int kRowChunks = kTile * 2 / 16;
#pragma unroll 4
  for (int q = int(threadIdx.x); q < kTile * kRowChunks; q += kT) {
    const int vl = q / kRowChunks, ch = q % kRowChunks;
    const int64_t v = v0 + vl, n = n0 + ch * 8;
    if (v < c.cpad && n < c.npad)
      *reinterpret_cast<uint4*>(c.g_cn + v * c.nld + n) =
          *reinterpret_cast<const uint4*>(tg + vl * kTile + ch * 8);
  }
}

enum DhMode { kDhOnly = 0, kDhFirst = 1, kDhMiddle = 2, kDhLast = 3 };

// Four dh values (consecutive columns) to bf16, as one 8-byte store when the
// output is 8-byte aligned, else one 2-byte store each.
RLK_DEV void store_bf16x4(uint16_t* p, float x, float y, float z, float w, bool vec) {
  const uint16_t b0 = to_bf16(x), b1 = to_bf16(y), b2 = to_bf16(z), b3 = to_bf16(w);
  if (vec) {
    *reinterpret_cast<uint2*>(p) = make_uint2(uint32_t(b0) | (uint32_t(b1) << 16),
                                              uint32_t(b2) | (uint32_t(b3) << 16));
  } else {
    p[0] = b0;
    p[1] = b1;
    p[2] = b2;
    p[3] = b3;
  }
}

// dh tile (tokens x hidden columns) += G_c W_c over the chunk's vocabulary.
// Each wave passes its 128 x 128 block through LDS one 32-column slab at a
// time (16 KB per wave), so a lane reads and writes four consecutive columns
// of a dh row at once: 16-byte fp32 partial sums (all 16 of a slab's loads
// issued before the adds) and 8-byte bf16 outputs.
template <int kMode>
__global__ __launch_bounds__(kT) void bwd_dh_tile(FusedBwdArgs a, ChunkArgs c) {
  __shared__ gemm::Smem smem;
  const int nnt = int((a.N + kTile - 1) / kTile), nht = int((a.H + kTile - 1) / kTile);
  int nt, ht;
  gemm::tile_of_block(nnt, nht, nt, ht);
  const int64_t n0 = int64_t(nt) * kTile, k0 = int64_t(ht) * kTile;
  f32x16 acc[4][4];
  gemm::gemm_nt_tile(acc, smem, c.g_nc, n0, a.N, c.cap, c.wt + c.c0, k0, a.H, c.vld, c.cpad);

  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  float* stg = reinterpret_cast<float*>(&smem[0][0][0]) + wid * (128 * 32);
  const bool vec_out = (reinterpret_cast<uintptr_t>(a.dh) & 7u) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // acc[i][j][r] is token 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4, column 32 j + lane % 32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stg[(32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * 32 + (lane & 31)] =
            acc[i][j][r];
    __syncthreads();
    // lane: columns col .. col + 3 (H is a multiple of 64, so all or none
    // exist) of tokens n0 + 128 wm + 8 q + lane / 8
    const int64_t col = k0 + 128 * wn + 32 * j + 4 * (lane & 7);
    f32x4 prev[16];
    if (kMode == kDhMiddle || kMode == kDhLast) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t n = n0 + 128 * wm + 8 * q + (lane >> 3);
        prev[q] = (n < a.N && col < a.H)
                      ? *reinterpret_cast<const f32x4*>(c.dh_acc + n * a.H + col)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int tl = 8 * q + (lane >> 3);
      const int64_t n = n0 + 128 * wm + tl;
      f32x4 v = *reinterpret_cast<const f32x4*>(stg + tl * 32 + 4 * (lane & 7));
      if (n >= a.N || col >= a.H) continue;
      const int64_t o = n * a.H + col;
      if (kMode == kDhMiddle || kMode == kDhLast) v = prev[q] + v;
      if (kMode == kDhFirst || kMode == kDhMiddle)
        *reinterpret_cast<f32x4*>(c.dh_acc + o) = v;
      else
        store_bf16x4(a.dh + o, v[0], v[1], v[2], v[3], vec_out);
    }
    __syncthreads();
  }
}

// dW tile (chunk vocabulary rows x hidden columns) = G_c^T h over all tokens.
__global__ __launch_bounds__(kT) void bwd_dw_tile(FusedBwdArgs a, ChunkArgs c) {
  __shared__ gemm::Smem smem;
  const int nvt = int((c.csz + kTile - 1) / kTile), nht = int((a.H + kTile - 1) / kTile);
  int vt, ht;
  gemm::tile_of_block(nvt, nht, vt, ht);
  const int64_t v0 = int64_t(vt) * kTile, k0 = int64_t(ht) * kTile;
  f32x16 acc[4][4];
  gemm::gemm_nt_tile(acc, smem, c.g_cn, v0, c.csz, c.nld, c.ht, k0, a.H, c.nld, c.npad);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = k0 + gemm::acc_b_row(j);
    if (col >= a.H) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t v = v0 + gemm::acc_a_row(i, r);
        if (v < c.csz) a.dW[(c.c0 + v) * a.H + col] = acc[i][j][r];
      }
  }
}

struct BwdLayout {
  int64_t npad, nld, vld, cap, nchunks;
  size_t off_wt, off_ht, off_gnc, off_gcn, off_acc, total;
};

BwdLayout bwd_layout(int64_t N, int64_t H, int64_t V) {
  BwdLayout L{};
  L.npad = round_up(N > 0 ? N : 1, 64);
  L.nld = L.npad + kLdPad;
  const int64_t vpad = round_up(V, 64);
  L.vld = vpad + kLdPad;
  L.cap = (vpad < kBwdChunk ? vpad : kBwdChunk) + kLdPad;
  L.nchunks = (V + kBwdChunk - 1) / kBwdChunk;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) / 256 * 256;
    return at;
  };
  L.off_wt = take(size_t(H) * size_t(L.vld) * 2);
  L.off_ht = take(size_t(H) * size_t(L.nld) * 2);
  L.off_gnc = take(size_t(N) * size_t(L.cap) * 2);
  L.off_gcn = take(size_t(L.cap) * size_t(L.nld) * 2);
  L.off_acc = take(L.nchunks > 1 ? size_t(N) * size_t(H) * 4 : 0);
  L.total = o;
  return L;
}

}  // namespace

size_t fused_bwd_workspace(int64_t N, int64_t H, int64_t V) { return bwd_layout(N, H, V).total; }

hipError_t launch_fused_bwd(const FusedBwdArgs& a, void* workspace, hipStream_t stream) {
  if (a.N == 0) {   // no tokens: dW = 0, dh is empty
    const int64_t n = a.V * a.H;
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    hipLaunchKernelGGL(fill_f32, dim3(unsigned(blocks)), dim3(256), 0, stream, a.dW, n);
    return hipGetLastError();
  }
  const BwdLayout L = bwd_layout(a.N, a.H, a.V);
  char* ws = reinterpret_cast<char*>(workspace);
  ChunkArgs c{};
  c.cap = L.cap;
  c.npad = L.npad;
  c.nld = L.nld;
  c.vld = L.vld;
  c.g_nc = reinterpret_cast<uint16_t*>(ws + L.off_gnc);
  c.g_cn = reinterpret_cast<uint16_t*>(ws + L.off_gcn);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + L.off_wt);
  uint16_t* ht = reinterpret_cast<uint16_t*>(ws + L.off_ht);
  c.wt = wt;
  c.ht = ht;
  c.dh_acc = reinterpret_cast<float*>(ws + L.off_acc);

  hipLaunchKernelGGL(transpose_pad, dim3(unsigned(L.vld / 64), unsigned(a.H / 64)), dim3(256), 0,
                     stream, a.w, a.V, a.ws, wt, L.vld);
  hipLaunchKernelGGL(transpose_pad, dim3(unsigned(L.nld / 64), unsigned(a.H / 64)), dim3(256), 0,
                     stream, a.h, a.N, a.hs, ht, L.nld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t nnt = (a.N + kTile - 1) / kTile, nht = (a.H + kTile - 1) / kTile;
  for (int64_t k = 0; k < L.nchunks; ++k) {
    c.c0 = k * kBwdChunk;
    c.csz = a.V - c.c0 < kBwdChunk ? a.V - c.c0 : kBwdChunk;
    c.cpad = round_up(c.csz, 64);
    const int64_t nvt = (c.csz + kTile - 1) / kTile;
    hipLaunchKernelGGL(bwd_g_tile, dim3(unsigned(nvt * nnt)), dim3(kT), 0, stream, a, c);
    const dim3 gdh(unsigned(nnt * nht));
    if (L.nchunks == 1)
      hipLaunchKernelGGL(bwd_dh_tile<kDhOnly>, gdh, dim3(kT), 0, stream, a, c);
    else if (k == 0)
      hipLaunchKernelGGL(bwd_dh_tile<kDhFirst>, gdh, dim3(kT), 0, stream, a, c);
    else if (k + 1 < L.nchunks)
      hipLaunchKernelGGL(bwd_dh_tile<kDhMiddle>, gdh, dim3(kT), 0, stream, a, c);
    else
      hipLaunchKernelGGL(bwd_dh_tile<kDhLast>, gdh, dim3(kT), 0, stream, a, c);
    hipLaunchKernelGGL(bwd_dw_tile, dim3(unsigned(nvt * nht)), dim3(kT), 0, stream, a, c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rlk
