// Fused LM head: token log-probability and entropy under softmax(h W^T / T)
// without materialising the [N, V] logits (prime-rl v0.10.0 release notes,
// "1. Trainer Performance": the loss is chunked torchtitan-style).
//
// Forward, two launches:
//  1. fwd_tile_stats: one block per (256-vocab x 256-token) tile. bf16 MFMA
//     (v_mfma_f32_32x32x16_bf16) accumulates z = W h^T in fp32 over the hidden
//     dimension, K staged through double-buffered, XOR-swizzled LDS. The
//     epilogue folds the tile's 256 logits of each token into a partial
//     (max z, sum 2^x, sum 2^x x) with x = (z - max) log2(e)/T, and the block
//     whose vocabulary slice holds a token's target writes that target logit.
//  2. fwd_merge: per token, the ceil(V/256) partials are merged in vocabulary
//     order in fp64 (a fixed order that depends on V only, so results do not
//     depend on the number of tokens or their order: the Qwen3-8B VIME
//     consistency page, "Canonical topology strategy", combines vocabulary
//     shards in one fixed order).
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "fused_kernels.h"

namespace rlk {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // vocabulary rows per block
constexpr int kBN = 256;   // tokens per block
constexpr int kBK = 64;    // hidden elements per stage
constexpr int kT = 256;    // threads per block: 2 x 2 waves of 128 x 128
constexpr int kChunks = kBK / 8;               // 16-byte chunks per staged row
constexpr int kLoadsPerThread = kBM * kChunks / kT;   // 8 per operand

constexpr float kLn2 = 0.6931471805599453f;

// LDS tile: [row][chunk], chunk index XOR-swizzled by (row & 7) so that the
// 32 rows an MFMA fragment read touches spread over all banks.
RLK_DEV int swz(int row, int chunk) { return row * kChunks + (chunk ^ (row & 7)); }

// Stage one kBK-wide slice of `rows` rows (starting at row0, clamped to
// [0, nrows)) of a [nrows, stride] bf16 matrix into registers.
RLK_DEV void load_slice(uint4 (&r)[kLoadsPerThread], const uint16_t* base, int64_t row0,
                        int64_t nrows, int64_t stride, int64_t k0) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int c = int(threadIdx.x) + i * kT;
    const int row = c / kChunks, ch = c % kChunks;
    const int64_t g = row0 + row;
    if (g < nrows)
      r[i] = *reinterpret_cast<const uint4*>(base + g * stride + k0 + ch * 8);
    else
      r[i] = make_uint4(0, 0, 0, 0);
  }
}

RLK_DEV void store_slice(uint4* lds, const uint4 (&r)[kLoadsPerThread]) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int c = int(threadIdx.x) + i * kT;
    lds[swz(c / kChunks, c % kChunks)] = r[i];
  }
}

// Merge of softmax partials (max m in z units, A = sum 2^x, B = sum 2^x x with
// x in log2 units of the scaled logit). c2 = log2(e)/T.
struct Part {
  float m, A, B;
};

RLK_DEV Part merge_part(Part p, Part q, float c2) {
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
  Part mine[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = vbase + 32 * i + 8 * (r >> 2) + 4 * fgrp + (r & 3);
        if (full || row < a.V) mx = fmaxf(mx, acc[i][j][r]);
      }
    float A = 0.f, B = 0.f;
    if (mx > -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = vbase + 32 * i + 8 * (r >> 2) + 4 * fgrp + (r & 3);
          if (full || row < a.V) {
            const float x = (acc[i][j][r] - mx) * c2;
            const float e = exp2f(x);
            A += e;
            B = fmaf(e, x, B);
          }
        }
    }
    Part p{mx, A, B};
    Part q;
    q.m = __shfl_xor(p.m, 32, 64);
    q.A = __shfl_xor(p.A, 32, 64);
    q.B = __shfl_xor(p.B, 32, 64);
    // lanes l and l^32 hold the same token: merge the lower half first
    mine[j] = fgrp == 0 ? merge_part(p, q, c2) : merge_part(q, p, c2);

    // target logit: the lane holding vocab row y of this token writes it
    const int64_t n = n0 + 128 * wn + 32 * j + frow;
    const int64_t y = n < a.N ? a.targets[n] : -1;
    const int64_t rel = y - vbase;
    const bool hit = rel >= 0 && rel < 128 && ((rel >> 2) & 1) == fgrp;
    if (__any(hit)) {
      const int ii = int(rel >> 5), ww = int(rel & 31);
      const int rr = ((ww >> 3) << 2) | (ww & 3);
      float val = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (i == ii && r == rr) val = acc[i][j][r];
      if (hit) a.zy[n] = val;
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
  __shared__ uint4 lds[2][2][kBM * kChunks];   // [buffer][A=W / B=h][swizzled tile]

  const int nnt = int((a.N + kBN - 1) / kBN);
  const int vt = int(blockIdx.x) / nnt, nt_blk = int(blockIdx.x) % nnt;
  const int64_t v0 = int64_t(vt) * kBM, n0 = int64_t(nt_blk) * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;   // wave's 128-row vocab half / 128-token half

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = int(a.H / kBK);
  uint4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  load_slice(ra, a.w, v0, a.V, a.ws, 0);
  load_slice(rb, a.h, n0, a.N, a.hs, 0);
  store_slice(lds[0][0], ra);
  store_slice(lds[0][1], rb);
  __syncthreads();

  const int frow = lane & 31, fgrp = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_slice(ra, a.w, v0, a.V, a.ws, int64_t(kt + 1) * kBK);
      load_slice(rb, a.h, n0, a.N, a.hs, int64_t(kt + 1) * kBK);
    }
    const uint4* As = lds[buf][0];
    const uint4* Bs = lds[buf][1];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = 2 * kk + fgrp;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 x = As[swz(128 * wm + 32 * i + frow, ch)];
        af[i] = __builtin_bit_cast(bf16x8, x);
        const uint4 y = Bs[swz(128 * wn + 32 * i + frow, ch)];
        bfr[i] = __builtin_bit_cast(bf16x8, y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_slice(lds[buf ^ 1][0], ra);
      store_slice(lds[buf ^ 1][1], rb);
    }
    __syncthreads();
  }

  tile_epilogue(a, acc, v0, n0, vt, reinterpret_cast<float*>(&lds[0][0][0]));
}

// ---------------------------------------------------------------------------
// Pipelined tile kernel. Each 64-wide slice of W and h goes global ->
// registers -> LDS: the loads of slice s+1 are issued before slice s is
// multiplied and written to the other LDS buffer after it, one barrier per
// slice. Inside a slice the fragments of k-step kk+1 are read from LDS while
// the 16 MFMAs of k-step kk run. Rows past the end are clamped to the last
// row (no branches in the load path); the epilogue masks their results.
// ---------------------------------------------------------------------------
// Per-thread element offsets (row * stride + chunk * 8) of the 8 chunks this
// thread stages from a [nrows, stride] matrix, rows clamped to the last one.
// 32-bit: the host routes matrices of 2^31 elements or more elsewhere.
RLK_DEV void slice_offsets(uint32_t (&off)[kLoadsPerThread], int64_t row0, int64_t nrows,
                           int64_t stride) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int c = int(threadIdx.x) + i * kT;
    int64_t g = row0 + c / kChunks;
    g = g < nrows ? g : nrows - 1;
    off[i] = uint32_t(g * stride + (c % kChunks) * 8);
  }
}

RLK_DEV void load_slice_off(uint4 (&r)[kLoadsPerThread], const uint16_t* base_k,
                            const uint32_t (&off)[kLoadsPerThread]) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i)
    r[i] = *reinterpret_cast<const uint4*>(base_k + off[i]);
}

RLK_DEV void read_frags(bf16x8 (&af)[4], bf16x8 (&bfr)[4], const uint4* As, const uint4* Bs,
                        int wm, int wn, int frow, int ch) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    af[i] = __builtin_bit_cast(bf16x8, As[swz(128 * wm + 32 * i + frow, ch)]);
    bfr[i] = __builtin_bit_cast(bf16x8, Bs[swz(128 * wn + 32 * i + frow, ch)]);
  }
}

RLK_DEV void mma_stage(f32x16 (&acc)[4][4], const uint4* As, const uint4* Bs, int wm, int wn,
                       int frow, int fgrp) {
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  read_frags(a0, b0, As, Bs, wm, wn, frow, fgrp);
#pragma unroll
  for (int kk = 0; kk < kBK / 16; kk += 2) {
    read_frags(a1, b1, As, Bs, wm, wn, frow, 2 * (kk + 1) + fgrp);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
    if (kk + 2 < kBK / 16) read_frags(a0, b0, As, Bs, wm, wn, frow, 2 * (kk + 2) + fgrp);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kT) void fwd_tile_stats_pipe(FusedFwdArgs a) {
  __shared__ uint4 LA[2][kBM * kChunks], LB[2][kBN * kChunks];

  const int nnt = int((a.N + kBN - 1) / kBN);
  const int vt = int(blockIdx.x) / nnt, nt_blk = int(blockIdx.x) % nnt;
  const int64_t v0 = int64_t(vt) * kBM, n0 = int64_t(nt_blk) * kBN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1, frow = lane & 31, fgrp = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = int(a.H / kBK);
  uint32_t oa[kLoadsPerThread], ob[kLoadsPerThread];
  slice_offsets(oa, v0, a.V, a.ws);
  slice_offsets(ob, n0, a.N, a.hs);
  uint4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  load_slice_off(ra, a.w, oa);
  load_slice_off(rb, a.h, ob);
  store_slice(LA[0], ra);
  store_slice(LB[0], rb);
  __syncthreads();

  for (int s = 0; s + 1 < nk; ++s) {
    const int buf = s & 1;
    // slice s+1 in flight while slice s is multiplied
    load_slice_off(ra, a.w + int64_t(s + 1) * kBK, oa);
    load_slice_off(rb, a.h + int64_t(s + 1) * kBK, ob);
    mma_stage(acc, LA[buf], LB[buf], wm, wn, frow, fgrp);
    store_slice(LA[buf ^ 1], ra);
    store_slice(LB[buf ^ 1], rb);
    __syncthreads();
  }
  mma_stage(acc, LA[(nk - 1) & 1], LB[(nk - 1) & 1], wm, wn, frow, fgrp);
  __syncthreads();
  tile_epilogue(a, acc, v0, n0, vt, reinterpret_cast<float*>(&LA[0][0]));
}

// ---------------------------------------------------------------------------
// LDS-DMA tile kernel. 32-wide hidden slices ("stages") of W and h are copied
// global -> LDS by global_load_lds_dwordx4 (no register staging). Five stage
// buffers (160 KB): while stage s is multiplied, stage s+1 is read into
// fragment registers and up to three later stages are in flight. Copies are
// issued two stages at a time (s+4 and s+5 at even steps), interleaved, so
// the two 64-byte halves of each 128-byte line of a row are requested
// together. One barrier per stage, preceded by an explicit vmcnt wait for
// this wave's copies of the next stage (the copies are invisible to the
// compiler's wait-count tracking, so every wait on them is written out here).
// Byte offsets are 32-bit: matrices of 2^32 bytes or more take fwd_tile_stats.
// ---------------------------------------------------------------------------
constexpr int kDK = 32;                     // hidden elements per stage
constexpr int kDStages = 5;                 // stage buffers resident in LDS
constexpr int kDChunks = kDK / 8;           // 16-byte chunks per staged row
constexpr int kDOpSlots = kBM * kDChunks;   // 16-byte slots per operand per stage
constexpr int kDLoads = kDOpSlots / kT;     // copies per thread per operand per stage
constexpr int kDVm = 2 * kDLoads;           // vmcnt of one stage (W and h)

// Physical chunk of (row, logical chunk): XOR with a 2-bit hash of the row so
// that both 8- and 16-lane groups of a 32-row fragment read hit distinct
// 16-byte bank groups.
RLK_DEV int dswz(int row) { return ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1); }
RLK_DEV int dslot(int row, int lc) { return row * kDChunks + (lc ^ dswz(row)); }

// Byte offsets of this thread's copies: copy j of wave w fills slots
// [64 q, 64 q + 64) with q = w * kDLoads + j, lane l writing slot 64 q + l.
RLK_DEV void dma_offsets(uint32_t (&off)[kDLoads], int64_t row0, int64_t nrows, int64_t stride) {
  const int w = int(threadIdx.x) >> 6, lane = int(threadIdx.x) & 63;
#pragma unroll
  for (int j = 0; j < kDLoads; ++j) {
    const int slot = (w * kDLoads + j) * 64 + lane;
    const int row = slot / kDChunks, lc = (slot % kDChunks) ^ dswz(row);
    int64_t g = row0 + row;
    g = g < nrows ? g : nrows - 1;
    off[j] = uint32_t((g * stride + lc * 8) * 2);
  }
}

// Copies of stages t and t+1 (64-byte halves of the same rows), interleaved.
RLK_DEV void dma_issue_pair(uint4* lds_t, uint4* lds_t1, const uint16_t* gbase_t,
                            const uint32_t (&off)[kDLoads]) {
  const int w = int(threadIdx.x) >> 6;
  const uint16_t* gbase_t1 = gbase_t + kDK;
#pragma unroll
  for (int j = 0; j < kDLoads; ++j) {
    const uint32_t m0a = uint32_t(reinterpret_cast<uintptr_t>(lds_t + (w * kDLoads + j) * 64));
    const uint32_t m0b = uint32_t(reinterpret_cast<uintptr_t>(lds_t1 + (w * kDLoads + j) * 64));
    asm volatile(
        "s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %4"
        :
        : "s"(__builtin_amdgcn_readfirstlane(m0a)), "s"(__builtin_amdgcn_readfirstlane(m0b)),
          "v"(off[j]), "s"(gbase_t), "s"(gbase_t1)
        : "memory", "m0");
  }
}

// Wait until at most N of this wave's vector-memory operations (here: LDS
// copies) are outstanding and its LDS reads are done, then barrier.
template <int N>
RLK_DEV void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

struct Frags {
  bf16x8 a[2][4], b[2][4];   // [k-step][32-row group]
};

// Fragment rows 128 wm + 32 x + frow: the swizzle hash depends on row & 15
// = frow & 15 only, so a read's address is a per-lane part (one per k-step)
// plus a uniform part.
struct FragAddr {
  uint32_t lane_off[2];   // bytes, per k-step
  uint32_t a_off, b_off;  // bytes: the wave's W rows and h rows inside a stage
};

RLK_DEV FragAddr frag_addr(int wm, int wn, int frow, int fgrp) {
  FragAddr f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) f.lane_off[kk] = uint32_t(dslot(frow, 2 * kk + fgrp)) * 16u;
  f.a_off = uint32_t(128 * wm * kDChunks * 16);
  f.b_off = uint32_t(kDOpSlots * 16 + 128 * wn * kDChunks * 16);
  return f;
}

RLK_DEV void read_frag(Frags& f, int r, const char* stage, const FragAddr& fa) {
  const int kk = r >> 3, x = r & 7;
  if (x < 4)
    f.a[kk][x] = *reinterpret_cast<const bf16x8*>(stage + fa.a_off + fa.lane_off[kk] +
                                                  x * 32 * kDChunks * 16);
  else
    f.b[kk][x - 4] = *reinterpret_cast<const bf16x8*>(stage + fa.b_off + fa.lane_off[kk] +
                                                      (x - 4) * 32 * kDChunks * 16);
}

// The 32 MFMAs of one stage; with kRead the 16 fragment reads of the next
// stage are interleaved with the first 16 MFMAs, so they have landed before
// the barrier that ends the stage.
template <bool kRead>
RLK_DEV void stage_mma(f32x16 (&acc)[4][4], const Frags& cur, Frags& nxt, const char* stage,
                       const FragAddr& fa) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[kk][i], cur.b[kk][j], acc[i][j],
                                                            0, 0, 0);
        const int m = kk * 16 + i * 4 + j;
        if (kRead && m < 16) {
          read_frag(nxt, m, stage, fa);
          // keep the issue order as written: the scheduler would otherwise
          // sink the reads to their uses in the next stage
          __builtin_amdgcn_sched_barrier(0);
        }
      }
}

constexpr int kDStageBytes = 2 * kDOpSlots * 16;   // 32 KB: W then h
constexpr int kXcds = 8;      // workgroups are dealt to the XCDs round-robin
constexpr int kGroupVt = 8;   // vocabulary tiles per group of the tile order

// Tile of a workgroup. Each XCD takes a contiguous range of the tile order,
// so its L2 serves one region of W and h; within the order, groups of
// kGroupVt vocabulary tiles sweep all token tiles with the vocabulary tile
// fastest, so the 32 workgroups an XCD runs at once cover about 8 W tiles
// and 4 h tiles.
RLK_DEV void tile_of_block(int nvt, int nnt, int& vt, int& nt) {
  const int T = nvt * nnt, b = int(blockIdx.x);
  const int x = b % kXcds, q = T / kXcds, r = T % kXcds;
  const int lid = x * q + (x < r ? x : r) + b / kXcds;
  const int grp = lid / (kGroupVt * nnt), rem = lid % (kGroupVt * nnt);
  const int gv = kGroupVt < nvt - grp * kGroupVt ? kGroupVt : nvt - grp * kGroupVt;
  vt = grp * kGroupVt + rem % gv;
  nt = rem / gv;
}

__global__ __launch_bounds__(kT) void fwd_tile_stats_dma(FusedFwdArgs a) {
  __shared__ uint4 smem[kDStages][2][kDOpSlots];   // [stage][W, h][slot]: 128 KB
  const char* sbase = reinterpret_cast<const char*>(&smem[0][0][0]);

  const int nnt = int((a.N + kBN - 1) / kBN);
  int vt, nt_blk;
  tile_of_block(int(gridDim.x) / nnt, nnt, vt, nt_blk);
  const int64_t v0 = int64_t(vt) * kBM, n0 = int64_t(nt_blk) * kBN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1, frow = lane & 31, fgrp = lane >> 5;
  const FragAddr fa = frag_addr(wm, wn, frow, fgrp);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // nk is even (the hidden size is a multiple of 64). Copies past the end
  // repeat the last stage into buffers no later step reads, so the wait
  // counts are the same at every step.
  const int nk = int(a.H / kDK);
  uint32_t oa[kDLoads], ob[kDLoads];
  dma_offsets(oa, v0, a.V, a.ws);
  dma_offsets(ob, n0, a.N, a.hs);
  auto issue_pair = [&](int t) __attribute__((always_inline)) {   // stages t, t+1 (t even)
    const int64_t k0 = int64_t(t < nk ? t : nk - 2) * kDK;
    dma_issue_pair(smem[t % kDStages][0], smem[(t + 1) % kDStages][0], a.w + k0, oa);
    dma_issue_pair(smem[t % kDStages][1], smem[(t + 1) % kDStages][1], a.h + k0, ob);
  };
  issue_pair(0);
  issue_pair(2);
  vm_wait_barrier<3 * kDVm>();
  Frags f0, f1;
#pragma unroll
  for (int r = 0; r < 16; ++r) read_frag(f0, r, sbase, fa);

  // Step s: stage s (fragments in registers) is multiplied while stage s+1
  // is read. Even s: after the barrier (stage s+1 landed; stages s-1 and s
  // consumed) stages s+4 and s+5 are copied into the buffers of s-1 and s.
  for (int s = 0; s < nk; s += 2) {
    vm_wait_barrier<2 * kDVm>();   // in flight: s+2, s+3
    issue_pair(s + 4);
    stage_mma<true>(acc, f0, f1, sbase + ((s + 1) % kDStages) * kDStageBytes, fa);
    vm_wait_barrier<3 * kDVm>();   // in flight: s+3, s+4, s+5
    stage_mma<true>(acc, f1, f0, sbase + ((s + 2) % kDStages) * kDStageBytes, fa);
  }
  vm_wait_barrier<0>();
  tile_epilogue(a, acc, v0, n0, vt, reinterpret_cast<float*>(&smem[0][0][0]));
}

__global__ __launch_bounds__(256) void fwd_merge(FusedFwdArgs a, int nvt) {
  const int64_t n = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (n >= a.N) return;
  const double c2 = double(a.c2);
  double m = -INFINITY, A = 0.0, B = 0.0;   // B in log2 units
  for (int vt = 0; vt < nvt; ++vt) {
    const float4 p = a.part[int64_t(vt) * a.N + n];
    if (double(p.x) == -INFINITY) continue;
    const double pm = p.x;
    if (m == -INFINITY) {
      m = pm;
      A = p.y;
      B = p.z;
      continue;
    }
    const double mm = pm > m ? pm : m;
    const double d1 = (m - mm) * c2, d2 = (pm - mm) * c2;
    const double s1 = exp2(d1), s2 = exp2(d2);
    B = s1 * (B + d1 * A) + s2 * (double(p.z) + d2 * double(p.y));
    A = A * s1 + double(p.y) * s2;
    m = mm;
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
  a.logprob[n] = lp;
  a.entropy[n] = float(H);
  if (a.saved) {
    a.saved[4 * n + 0] = float(m * invT + lnA);   // log Z of the scaled logits z/T
    a.saved[4 * n + 1] = float(m * invT + Ed);    // E_q[z/T]
    a.saved[4 * n + 2] = -INFINITY;              // no cut at top-p = 1
    a.saved[4 * n + 3] = 0.f;
  }
  if (a.nsize) a.nsize[n] = int32_t(a.V);
  if (a.flags) a.flags[n] = flags;
}

}  // namespace

size_t fused_fwd_workspace(int64_t N, int64_t H, int64_t V) {
  (void)H;
  const int64_t nvt = (V + kBM - 1) / kBM;
  return size_t(nvt * N) * 16 + size_t(N) * 4 + 512;
}

hipError_t launch_fused_fwd(FusedFwdArgs a, void* workspace, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  const int64_t nvt = (a.V + kBM - 1) / kBM, nnt = (a.N + kBN - 1) / kBN;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part = reinterpret_cast<float4*>(ws);
  a.zy = reinterpret_cast<float*>(ws + (size_t(nvt * a.N) * 16 + 255) / 256 * 256);
  if (a.V * a.ws < (int64_t(1) << 31) && a.N * a.hs < (int64_t(1) << 31) && a.H % kDK == 0)
    hipLaunchKernelGGL(fwd_tile_stats_dma, dim3(unsigned(nvt * nnt)), dim3(kT), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_tile_stats, dim3(unsigned(nvt * nnt)), dim3(kT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_merge, dim3(unsigned((a.N + 255) / 256)), dim3(256), 0, stream, a,
                     int(nvt));
  return hipGetLastError();
}

}  // namespace rlk
