// Device-side core of the fused LM-head kernels: one 256 x 256 output tile
// of C = A B^T with bf16 operands whose K dimension is contiguous (row-major
// [rows, ld] matrices), accumulated in fp32 on v_mfma_f32_32x32x16_bf16.
//
// Block: 256 threads = 2 x 2 waves, each wave owning 128 A rows x 128 B rows
// as 4 x 4 MFMA blocks of 32 x 32 (acc[i][j], 256 accumulator registers).
// After gemm_nt_tile, acc[i][j][r] holds
//   A row  a_row0 + 128 wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
//   B row  b_row0 + 128 wn + 32 j + lane % 32,
// with wm = wave / 2, wn = wave % 2. Rows past the end of A or B are clamped
// to the last row when loading (no branches); their results must be masked.
//
// K streams through LDS in 32-wide stages copied global -> LDS by
// global_load_lds_dwordx4 (no register staging). Five stage buffers
// (5 x 32 KB = 160 KB): while stage s is multiplied, stage s+1 is read into
// fragment registers and up to three later stages are in flight. Copies are
// issued two stages at a time (s+4 and s+5 at even steps), interleaved, so
// the two 64-byte halves of each 128-byte line of a row are requested
// together. One barrier per stage, preceded by an explicit vmcnt wait for
// this wave's copies of the next stage: the copies are inline assembly,
// invisible to the compiler's wait-count tracking, so every wait on them is
// written out here, and the loop issues the same number of copies at every
// step (past the end it repeats the last stages into buffers that no later
// step reads) so the wait counts are constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace rlk {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;                    // rows of A and of B per tile
constexpr int kThreads = 256;                 // 2 x 2 waves of 128 x 128
constexpr int kStageK = 32;                   // K elements per stage
constexpr int kStages = 5;                    // stage buffers resident in LDS
constexpr int kChunks = kStageK / 8;          // 16-byte chunks per staged row
constexpr int kOpSlots = kTile * kChunks;     // 16-byte slots per operand per stage
constexpr int kLoads = kOpSlots / kThreads;   // copies per thread per operand per stage
constexpr int kVmPerStage = 2 * kLoads;       // vmcnt of one stage (A and B)
constexpr int kStageBytes = 2 * kOpSlots * 16;  // 32 KB: A then B
constexpr int kKMultiple = 2 * kStageK;       // K must be a multiple of this
// largest row length (elements): a copy's per-lane byte offset, up to
// (255 ld + 24) 2, is a 32-bit unsigned value
constexpr int64_t kMaxLd = ((int64_t(1) << 32) - 48) / 510;

// LDS of one block: [stage][A, B][slot].
typedef uint4 Smem[kStages][2][kOpSlots];

// Physical chunk of (row, logical chunk): XOR with a 2-bit hash of the row so
// that both the 8- and the 16-lane groups of a 32-row fragment read hit
// distinct 16-byte bank groups.
RLK_DEV int swz_hash(int row) {
  return ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1);
}
RLK_DEV int slot_of(int row, int lc) { return row * kChunks + (lc ^ swz_hash(row)); }

// Byte offsets, relative to the tile's first row, of this thread's copies:
// copy j of wave w fills slots [64 q, 64 q + 64) with q = w * kLoads + j,
// lane l writing slot 64 q + l.
RLK_DEV void copy_offsets(uint32_t (&off)[kLoads], int64_t row0, int64_t nrows, int64_t ld) {
  const int w = int(threadIdx.x) >> 6, lane = int(threadIdx.x) & 63;
  const int last = int(nrows - 1 - row0 < kTile - 1 ? nrows - 1 - row0 : kTile - 1);
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int slot = (w * kLoads + j) * 64 + lane;
    const int row = slot / kChunks, lc = (slot % kChunks) ^ swz_hash(row);
    const int r = row < last ? row : last;
    off[j] = uint32_t((int64_t(r) * ld + lc * 8) * 2);
  }
}

// LDS addresses are 32-bit integers here. Everything a copy needs besides
// the per-lane global offset is uniform over the wave (its LDS destination
// goes to M0), so it is formed from scalar values only; formed from per-lane
// values it costs a VALU chain and a v_readfirstlane per copy, which in-order
// issue has to wait out between the MFMAs (about 8 % of the loop's time).
// Fragment reads use one per-lane base per operand and k-step plus the
// stage's offset, the rest as the instruction's immediate offset.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_frag;

struct TileCtx {
  uint32_t lds;          // LDS byte address of the stage buffers
  uint32_t wave_off;     // bytes: this wave's first copy slot inside an operand, w * kLoads * 1 KB
  uint32_t frag[2][2];   // per lane, [A, B][k-step]: LDS byte address of its fragment row in stage 0
};

// Fragment rows 128 wm + 32 x + lane % 32: the swizzle hash depends on
// row & 15 only, so a read's address is a per-lane part (one per k-step) plus
// a uniform part.
RLK_DEV TileCtx tile_ctx(Smem& smem) {
  TileCtx c;
  c.lds = uint32_t(reinterpret_cast<uintptr_t>((lds_char*)(&smem[0][0][0])));
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  c.wave_off = uint32_t(w * kLoads * 64 * 16);
  const int lane = int(threadIdx.x) & 63, wid = int(threadIdx.x) >> 6;
  const int wm = wid >> 1, wn = wid & 1, frow = lane & 31, fgrp = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint32_t lo = uint32_t(slot_of(frow, 2 * kk + fgrp)) * 16u;
    c.frag[0][kk] = c.lds + uint32_t(128 * wm * kChunks * 16) + lo;
    c.frag[1][kk] = c.lds + uint32_t(kOpSlots * 16 + 128 * wn * kChunks * 16) + lo;
  }
  return c;
}

// Copy unit u of a stage pair: operand u / kLoads, this thread's slot
// j = u % kLoads, of stages t and t+1 (buffers bt and bt1, global base g0 of
// stage t), the 64-byte halves of the same rows back to back. The copy reads
// its LDS destination from M0, which the statement sets and declares
// clobbered (clang warns that M0 is reserved; declaring it is what keeps the
// compiler from relying on an M0 value across the statement).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
RLK_DEV void copy_unit(const TileCtx& c, int u, int bt, int bt1, const uint16_t* g0,
                       const uint32_t (&oa)[kLoads], const uint32_t (&ob)[kLoads]) {
  const int op = u / kLoads, j = u % kLoads;
  const uint32_t m0a = c.lds + uint32_t(((bt * 2 + op) * kOpSlots + j * 64) * 16) + c.wave_off;
  const uint32_t m0b = c.lds + uint32_t(((bt1 * 2 + op) * kOpSlots + j * 64) * 16) + c.wave_off;
  const uint16_t* g1 = g0 + kStageK;
  asm volatile(
      "s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %4"
      :
      : "s"(m0a), "s"(m0b), "v"(op == 0 ? oa[j] : ob[j]), "s"(g0), "s"(g1)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory operations (here: LDS
// copies) are outstanding and its LDS reads are done, then barrier.
template <int N>
RLK_DEV void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

struct Frags {
  bf16x8 a[2][4], b[2][4];   // [k-step][32-row group]
};

// Fragment read r of a stage at byte offset stage_off: k-step r / 8, row
// group r % 8 (A for 0..3, B for 4..7).
RLK_DEV void read_frag(Frags& f, int r, uint32_t stage_off, const TileCtx& c) {
  const int kk = r >> 3, x = r & 7;
  if (x < 4) {
    lds_frag* p = reinterpret_cast<lds_frag*>(uintptr_t(c.frag[0][kk] + stage_off));
    f.a[kk][x] = p[x * 32 * kChunks];
  } else {
    lds_frag* p = reinterpret_cast<lds_frag*>(uintptr_t(c.frag[1][kk] + stage_off));
    f.b[kk][x - 4] = p[(x - 4) * 32 * kChunks];
  }
}

// Issue schedule inside a stage's 32 MFMAs (m = MFMA index): the 16
// fragment reads of the next stage go after MFMAs read_slot(r), and the
// stage's 4 copy units after MFMAs copy_slot(u), so that LDS reads and LDS
// copies are spread over the stage and the last read lands before the
// barrier that ends it.
constexpr int read_slot(int r) { return r; }
constexpr int copy_slot(int u) { return 16 + 4 * u; }

// The 32 MFMAs of one stage, the next stage's fragment reads (at byte offset
// next_off) and the copy units of operand kCopyOp (0 = A, 1 = B) of the
// stage pair in buffers bt, bt1 from global bases ga (A) / gb (B).
template <int kCopyOp>
RLK_DEV void stage_mma(f32x16 (&acc)[4][4], const Frags& cur, Frags& nxt, uint32_t next_off,
                       const TileCtx& c, int bt, int bt1, const uint16_t* ga, const uint16_t* gb,
                       const uint32_t (&oa)[kLoads], const uint32_t (&ob)[kLoads]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[kk][i], cur.b[kk][j], acc[i][j],
                                                            0, 0, 0);
        const int m = kk * 16 + i * 4 + j;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (read_slot(r) == m) read_frag(nxt, r, next_off, c);
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
          if (copy_slot(u) == m)
            copy_unit(c, kCopyOp * kLoads + u, bt, bt1, kCopyOp ? gb : ga, oa, ob);
        // keep the issue order as written: the scheduler would otherwise
        // sink the reads to their uses in the next stage
        __builtin_amdgcn_sched_barrier(0);
      }
}

// acc = A[a_row0 .. +256) . B[b_row0 .. +256)^T over k in [0, K); K is a
// positive multiple of kKMultiple. Ends with a barrier after which `smem` may
// be reused.
RLK_DEV void gemm_nt_tile(f32x16 (&acc)[4][4], Smem& smem, const uint16_t* A, int64_t a_row0,
                          int64_t a_rows, int64_t lda, const uint16_t* B, int64_t b_row0,
                          int64_t b_rows, int64_t ldb, int64_t K) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const TileCtx c = tile_ctx(smem);
  const int nk = int(K / kStageK);   // even
  uint32_t oa[kLoads], ob[kLoads];
  copy_offsets(oa, a_row0, a_rows, lda);
  copy_offsets(ob, b_row0, b_rows, ldb);
  const uint16_t* a_base = A + a_row0 * lda;
  const uint16_t* b_base = B + b_row0 * ldb;
  // global K offset of the pair t, t+1 (t even); past the end, the last pair
  auto kof = [&](int t) __attribute__((always_inline)) {
    return int64_t(t < nk ? t : nk - 2) * kStageK;
  };
#pragma unroll
  for (int t = 0; t < 4; t += 2)
#pragma unroll
    for (int u = 0; u < 2 * kLoads; ++u)
      copy_unit(c, u, t, t + 1, (u < kLoads ? a_base : b_base) + kof(t), oa, ob);
  vm_wait_barrier<2 * kVmPerStage>();   // stages 0 and 1 landed
  Frags f0, f1;
#pragma unroll
  for (int r = 0; r < 16; ++r) read_frag(f0, r, 0u, c);

  // Step s: stage s (fragments in registers) is multiplied while stage s+1
  // is read. Stages s+4 and s+5 are copied into the buffers of stages s-1
  // and s (both consumed before step s): operand A during step s, operand B
  // during step s+1 (s even). Copies complete in issue order, so at the top
  // of an even step the wait leaves the last 16 copies (pair s+2, s+3) in
  // flight and at the top of an odd step the last 8 (A of pair s+4, s+5).
  // b1, b2, b4: buffers of stages s+1, s+2, s+4.
  int b1 = 1, b2 = 2, b4 = 4;
  for (int s = 0; s < nk; s += 2) {
    vm_wait_barrier<2 * kVmPerStage>();   // stage s+1 landed
    const int b5 = b4 == kStages - 1 ? 0 : b4 + 1;
    const uint16_t* ga = a_base + kof(s + 4);
    const uint16_t* gb = b_base + kof(s + 4);
    stage_mma<0>(acc, f0, f1, uint32_t(b1 * kStageBytes), c, b4, b5, ga, gb, oa, ob);
    vm_wait_barrier<kVmPerStage>();       // stage s+2 landed
    stage_mma<1>(acc, f1, f0, uint32_t(b2 * kStageBytes), c, b4, b5, ga, gb, oa, ob);
    b1 = b1 + 2 >= kStages ? b1 + 2 - kStages : b1 + 2;
    b2 = b2 + 2 >= kStages ? b2 + 2 - kStages : b2 + 2;
    b4 = b4 + 2 >= kStages ? b4 + 2 - kStages : b4 + 2;
  }
  vm_wait_barrier<0>();
}

constexpr int kXcds = 8;      // workgroups are dealt to the XCDs round-robin
constexpr int kSupA = 32;     // A tiles per super-tile
constexpr int kSupB = 8;      // B tiles per super-tile
constexpr int kSubA = 8;      // A tiles of one XCD's part of a super-tile
constexpr int kSubB = 4;      // B tiles of one XCD's part
static_assert((kSupA / kSubA) * (kSupB / kSubB) == kXcds && kSubA * kSubB * kXcds == kSupA * kSupB,
              "a super-tile is one 8 x 4 part per XCD");

// Tile (ta, tb) of this workgroup in an na x nb grid. The order runs over
// super-tiles of 32 A-tiles x 8 B-tiles (256 tiles: one per CU), B fastest
// within a band of 32 A-tiles. Inside a full super-tile, the 32 workgroups
// that one XCD receives (every 8th) cover an 8 x 4 part of it. So the tiles
// that run at one time read 32 A and 8 B panels between them, which the
// memory-side cache holds, and each XCD's L2 serves 8 + 4 of them. A ragged
// super-tile (the last band or the end of a band) is taken A-fastest.
// The map is a bijection on [0, na nb) (checked on the host for many grids).
RLK_DEV void tile_of_block(int na, int nb, int& ta, int& tb) {
  const int b = int(blockIdx.x);
  const int band = b / (kSupA * nb), i = b % (kSupA * nb);
  const int ga = kSupA < na - band * kSupA ? kSupA : na - band * kSupA;
  const int blk = i / (ga * kSupB), j = i % (ga * kSupB);
  const int gb = kSupB < nb - blk * kSupB ? kSupB : nb - blk * kSupB;
  int a, c;
  if (ga == kSupA && gb == kSupB) {
    constexpr int kPartsA = kSupA / kSubA;
    const int x = j % kXcds, s = j / kXcds;
    a = (x % kPartsA) * kSubA + s % kSubA;
    c = (x / kPartsA) * kSubB + s / kSubA;
  } else {
    a = j % ga;
    c = j / ga;
  }
  ta = band * kSupA + a;
  tb = blk * kSupB + c;
}

// Row of acc[i][j][r] inside the A and B halves of the tile (see the top).
RLK_DEV int acc_a_row(int i, int r) {
  const int lane = int(threadIdx.x) & 63, wm = int(threadIdx.x) >> 7;
  return 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
RLK_DEV int acc_b_row(int j) {
  const int lane = int(threadIdx.x) & 63, wn = (int(threadIdx.x) >> 6) & 1;
  return 128 * wn + 32 * j + (lane & 31);
}

}  // namespace gemm
}  // namespace rlk
