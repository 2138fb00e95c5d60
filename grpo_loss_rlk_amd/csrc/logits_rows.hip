// Logits in: full and top-p truncated log-probability and entropy per row.
//
// What is computed (Qwen3-8B VIME train-rollout consistency page, "ROCm MI300X
// and gfx942": temperature > 0, top-p in (0, 1], the complete nucleus is
// scored, top-p = 1 is the full vocabulary, a monitoring entropy is fused
// with the logprob): for a row z, d_i = (z_i - max z)/T, the full softmax
// statistics, the nucleus S = {z >= tau} with tau the lowest row value whose
// strictly-higher mass is below p (all ties kept), and the statistics of the
// distribution renormalised over S. With the opt-in top-k, a first kernel
// (topk_floor_rows) finds each row's k-th largest value v_k and the cut then
// runs on the values >= v_k only, its masses relative to their sum (the
// prime-rl v0.10.0 release notes, "2. RL Algorithms", replay top-k in the
// trainer); at top-p 1 the nucleus is {z >= v_k}.
//
// Row kernels, chosen per call by dtype and vocabulary size only (never by
// the number of rows, so a row's result does not depend on its batch):
//
//  * bf16_hist_rows: bf16 rows with V >= 16384. A bf16 value has only 65536
//    bit patterns, so one streaming pass that counts each pattern in LDS
//    captures the whole row. Everything after that -- max, Z, entropy, the
//    top-p cut, the truncated sums -- is arithmetic over the distinct values
//    (fp32 masses, exact fixed-point sums), so HBM is read once at a few
//    VALU ops per element. The counters (16-bit, a positive and a negative
//    pattern per 32-bit word) cover the magnitudes with bf16 exponent field
//    0x40..0xbf, |z| in [2^-63, 2^64): 64 KB per buffer. Two buffers let 12
//    waves stream the next row while 4 waves post-process the previous
//    one. Zeros and -inf are tallied on the side; a row holding +inf, NaN,
//    extreme magnitudes or one value more than 65535 times is handed to the
//    generic kernel.
//
//  * f32_rows: fp32 rows (below).
//
//  * generic_rows: any dtype and size. Multi-pass over the row: max, then
//    exp / Z / entropy with a 12-bit radix histogram of fixed-point masses,
//    then two refinement rounds (10 + 10 bits) restricted to the boundary
//    bin, then the truncated sums. Masses are integers (2^-39 of the max
//    element's mass) so LDS atomics are order-free and the cut is bitwise
//    deterministic.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rlk {

namespace {

constexpr uint8_t kOutside = 1, kBadTarget = 2, kNonFinite = 4, kBoundary = 8, kBadParam = 16;
constexpr double kBoundaryEps = 1e-6;

RLK_DEV bool param_ok(float T, float p) {
  return T > 0.f && T <= 3.4e38f && p > 0.f && p <= 1.f;  // NaN fails every compare
}

// The row's top-k (0: off) and its floor v_k (-inf: no top-k cut).
RLK_DEV int32_t row_top_k(const RowArgs& a, int64_t row) {
  return a.k_row ? a.k_row[row] : a.top_k;
}
RLK_DEV float row_floor(const RowArgs& a, int64_t row) {
  return a.kfloor ? a.kfloor[row] : -INFINITY;
}

// lse_s, eq_s: log Z_S and E_q[z/T] over the nucleus, in units of z/T;
// the fused backward reads them, with tau and the lp-term flag, from saved4.
RLK_DEV void store_row(const RowArgs& a, int64_t row, float lp_full, float lp_trunc,
                       float h_full, float h_trunc, int32_t size, float tau, uint8_t flags,
                       float lse_s, float eq_s) {
  if (a.saved4) {   // slot 3: 1 when the row's lp term is live (target in range and kept)
    a.saved4[4 * row + 0] = lse_s;
    a.saved4[4 * row + 1] = eq_s;
    a.saved4[4 * row + 2] = tau;
    a.saved4[4 * row + 3] = (flags & (kOutside | kBadTarget | kNonFinite | kBadParam)) ? 0.f : 1.f;
  }
  a.lp_full[row] = lp_full;
  a.lp_trunc[row] = lp_trunc;
  a.ent_trunc[row] = h_trunc;
  if (a.ent_full) a.ent_full[row] = h_full;
  if (a.nsize) a.nsize[row] = size;
  if (a.thresh) a.thresh[row] = tau;
  if (a.flags) a.flags[row] = flags;
}

RLK_DEV void store_nan_row(const RowArgs& a, int64_t row, uint8_t flags) {
  const float nan = __builtin_nanf("");
  store_row(a, row, nan, nan, nan, nan, 0, nan, flags, nan, nan);
}

// ===========================================================================
// Generic radix-select kernel (fp32 or bf16 rows of any length)
// ===========================================================================
constexpr int kGT = 256;
constexpr int kBins1 = 4096;          // round 1: top 12 key bits
constexpr int kBins2 = 1024;          // rounds 2, 3: 10 bits each
constexpr double kFix = 549755813888.0;   // 2^39: fixed-point unit of mass (max element = 2^39)

template <typename T>
RLK_DEV float load_val(const T* p, int64_t i);
template <>
RLK_DEV float load_val<float>(const float* p, int64_t i) { return p[i]; }
template <>
RLK_DEV float load_val<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// exp((z - m) / T) in fp32 from an fp64 argument, and d = (z - m)/T in fp64
RLK_DEV float mass_of(float z, double m, double invT, double* d) {
  *d = (double(z) - m) * invT;
  return expf(float(*d));
}

RLK_DEV uint64_t fixed_mass(float e) { return uint64_t(double(e) * kFix + 0.5); }

// Walk `bins` from index `start` downward until carry + running sum >= thr.
// Returns the bin, or -1; *above receives the mass strictly above that bin.
template <int NT>
RLK_DEV int walk_down(const uint64_t* bins, int start, uint64_t thr, uint64_t carry,
                      uint64_t* above, uint64_t* su64, int* si, uint64_t* bslot) {
  for (int base = start; base >= 0; base -= NT) {
    const int b = base - int(threadIdx.x);
    const uint64_t v = b >= 0 ? bins[b] : 0ull;
    uint64_t tot;
    const uint64_t incl = block_inclusive_scan(v, su64, &tot);
    const int cand = (v != 0ull && carry + incl >= thr) ? int(threadIdx.x) : NT;
    const int first = block_min(cand, si);
    if (first < NT) {
      if (int(threadIdx.x) == first) *bslot = carry + incl - v;
      __syncthreads();
      *above = *bslot;
      __syncthreads();
      return base - first;
    }
    carry += tot;
  }
  *above = carry;
  return -1;
}

// LDS of the generic path: 4096 u64 bins plus reduction scratch.
struct GenScratch {
  uint64_t hist[kBins1];
  double sd[16];
  uint64_t su64[16];
  int si[16];
  float sf[16];
  uint64_t bslot;
};

// One row by the generic multi-pass algorithm, with a block of NT threads.
template <typename T, int NT>
RLK_DEV void generic_row(const RowArgs& a, int64_t row, GenScratch& g) {
  uint64_t* hist = g.hist;
  double* sd = g.sd;
  uint64_t* su64 = g.su64;
  int* si = g.si;
  float* sf = g.sf;
  uint64_t& bslot = g.bslot;
  const int tid = threadIdx.x;
  const int64_t V = a.vocab;
  const T* rowp = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;

  float Tv = a.t_row ? a.t_row[row] : a.temperature;
  float p = a.p_row ? a.p_row[row] : a.top_p;
  const int64_t y = a.targets[row];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  if (!param_ok(Tv, p) || row_top_k(a, row) < 0) {
    if (tid == 0) store_nan_row(a, row, flags | kBadParam);
    return;
  }
  // top-k: only values >= the floor take part in the cut (fk = 0: all)
  const float floor_v = row_floor(a, row);
  const bool has_floor = floor_v > -INFINITY;
  const uint32_t fk = has_floor ? f32_key(floor_v) : 0u;

  // ---- pass 1: max, finite count, non-finite detection ----
  float mx = -INFINITY;
  int bad = 0;
  uint32_t nfin = 0;
  for (int64_t i = tid; i < V; i += NT) {
    const float z = load_val(rowp, i);
    if (z != z || z == INFINITY) bad = 1;
    else if (z > -INFINITY) {
      mx = fmaxf(mx, z);
      ++nfin;
    }
  }
  mx = block_max(mx, sf);
  bad = block_max(bad, si);
  nfin = uint32_t(block_sum(uint64_t(nfin), su64));
  if (bad || nfin == 0) {
    if (tid == 0) store_nan_row(a, row, flags | kNonFinite);
    return;
  }
  const double m = double(mx);
  const double invT = 1.0 / double(Tv);
  const bool cut_p = p < 1.f;
  const bool cut = cut_p || has_floor;

  // ---- pass 2: Z, sum e*d, round-1 histogram of fixed-point masses (of
  //      the values at or above the top-k floor) ----
  for (int i = tid; i < kBins1; i += NT) hist[i] = 0ull;
  __syncthreads();
  double zt = 0.0, st = 0.0;
  uint64_t wt = 0;
  for (int64_t i = tid; i < V; i += NT) {
    const float z = load_val(rowp, i);
    if (!(z > -INFINITY)) continue;
    double d;
    const float e = mass_of(z, m, invT, &d);
    zt += double(e);
    st += double(e) * d;
    if (cut_p && f32_key(z) >= fk) {
      const uint64_t w = fixed_mass(e);
      if (w) {
        wt += w;
        atomicAdd(reinterpret_cast<unsigned long long*>(&hist[f32_key(z) >> 20]),
                  (unsigned long long)w);
      }
    }
  }
  const double Z = block_sum(zt, sd);
  const double S = block_sum(st, sd);

  double Zs = Z, Ss = S;
  uint32_t tau_key = 0;
  uint32_t size = nfin;
  if (cut) {
    if (cut_p) {
      const uint64_t W = block_sum(wt, su64);
      const uint64_t thr = uint64_t(ceil(double(p) * double(W)));
      // round 1
      uint64_t above = 0;
      int d1 = walk_down<NT>(hist, kBins1 - 1, thr, 0ull, &above, su64, si, &bslot);
      if (d1 < 0) d1 = 0;   // unreachable: the total mass reaches thr
      // round 2
      __syncthreads();
      for (int i = tid; i < kBins2; i += NT) hist[i] = 0ull;
      __syncthreads();
      for (int64_t i = tid; i < V; i += NT) {
        const float z = load_val(rowp, i);
        if (!(z > -INFINITY)) continue;
        const uint32_t k = f32_key(z);
        if (int(k >> 20) != d1 || k < fk) continue;
        double d;
        const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
        if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(k >> 10) & 0x3ffu]),
                         (unsigned long long)w);
      }
      __syncthreads();
      int d2 = walk_down<NT>(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
      if (d2 < 0) d2 = 0;
      // round 3
      __syncthreads();
      for (int i = tid; i < kBins2; i += NT) hist[i] = 0ull;
      __syncthreads();
      const uint32_t pre = (uint32_t(d1) << 10) | uint32_t(d2);
      for (int64_t i = tid; i < V; i += NT) {
        const float z = load_val(rowp, i);
        if (!(z > -INFINITY)) continue;
        const uint32_t k = f32_key(z);
        if ((k >> 10) != pre || k < fk) continue;
        double d;
        const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
        if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[k & 0x3ffu]),
                         (unsigned long long)w);
      }
      __syncthreads();
      int d3 = walk_down<NT>(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
      if (d3 < 0) d3 = 0;
      tau_key = (pre << 10) | uint32_t(d3);
      tau_key = tau_key > fk ? tau_key : fk;
      const uint64_t at = hist[d3];
      if (tid == 0) {
        const double pp = double(p);
        if (fabs(double(above) / double(W) - pp) <= kBoundaryEps ||
            fabs(double(above + at) / double(W) - pp) <= kBoundaryEps)
          flags |= kBoundary;
      }
    } else {
      tau_key = fk;   // top-k at top-p 1: S is the top-k set
    }
    // final pass: truncated sums over S = {key >= tau}
    double zs = 0.0, ss = 0.0;
    uint32_t cnt = 0;
    for (int64_t i = tid; i < V; i += NT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY) || f32_key(z) < tau_key) continue;
      double d;
      const float e = mass_of(z, m, invT, &d);
      zs += double(e);
      ss += double(e) * d;
      ++cnt;
    }
    Zs = block_sum(zs, sd);
    Ss = block_sum(ss, sd);
    size = uint32_t(block_sum(uint64_t(cnt), su64));
  }

  if (tid == 0) {
    const double logZ = log(Z), logZs = log(Zs);
    float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
    if (!(flags & kBadTarget)) {
      const float zy = load_val(rowp, y);
      if (!(zy > -INFINITY)) {
        lpf = -INFINITY;
        lpt = -INFINITY;
        flags |= kOutside;
      } else {
        lpf = token_logprob(zy, m, invT, logZ);
        if (!cut || f32_key(zy) >= tau_key) {
          lpt = token_logprob(zy, m, invT, logZs);
        } else {
          lpt = -INFINITY;
          flags |= kOutside;
        }
      }
    }
    const float tau = cut ? key_f32(tau_key) : -INFINITY;
    if (a.score_stats) {
      a.score_stats[2 * row] = m;
      a.score_stats[2 * row + 1] = logZs;
    }
    store_row(a, row, lpf, lpt, float(logZ - S / Z), float(logZs - Ss / Zs), int32_t(size), tau,
              flags, float(m * invT + logZs), float(m * invT + Ss / Zs));
  }
}


template <typename T>
__global__ __launch_bounds__(kGT) void generic_rows(RowArgs a) {
  __shared__ GenScratch g;
  generic_row<T, kGT>(a, int64_t(blockIdx.x), g);
}

// ===========================================================================
// bf16 pattern-count histogram kernel
// ===========================================================================
constexpr int kHT = 1024;                        // threads per block (one block per CU)
constexpr int kFW = 4;                           // finisher waves (one per SIMD)
constexpr int kStreamWaves = kHT / kWave - kFW;  // streaming waves
constexpr int kStreamers = kStreamWaves * kWave; // streaming threads
constexpr int kHWords = 16384;                   // 64 KB of 16-bit counter pairs per buffer
constexpr int kMagLo = 0x2000, kMagHi = 0x6000;  // counted magnitudes: |z| in [2^-63, 2^64)
constexpr int kKeyLo = 0x7fff - (kMagHi - 1);    // lowest merged key of a counted value
constexpr int kUnroll = 4;                       // 16-byte vectors in flight per streamer

// Counter index of a counted magnitude (a rotation of the window onto 0..16383).
RLK_DEV int widx(int mag) { return mag & 0x3fff; }
// Magnitude held by counter index i.
RLK_DEV int wmag(int i) { return i < 0x2000 ? i + 0x4000 : i; }

// One bf16 pattern: counted if its magnitude is in the window, else tallied
// as zero (+-0), -inf, or other (+inf, NaN, extreme magnitudes).
RLK_DEV void count_code(uint32_t* hist, uint32_t* special, uint32_t c) {
  const uint32_t mag = c & 0x7fffu;
  if (mag >= uint32_t(kMagLo) && mag < uint32_t(kMagHi))
    atomicAdd(&hist[mag & 0x3fffu], (c & 0x8000u) ? 0x10000u : 1u);
  else
    atomicAdd(&special[mag == 0 ? 0 : (c == 0xff80u ? 1 : 2)], 1u);
}

// Eight bf16 patterns (16 bytes). The counter pair at index magnitude & 0x3fff
// holds the positive pattern in its low half and the negative one in its
// high half. A pattern's magnitude is inside the window exactly when bit 14
// of (pattern + 0x2000), added in 16 bits, is set; when all eight pass that
// test (the normal case) they are counted directly, at a few operations per
// pattern: the counter's byte offset is a mask and a shift, and the
// increment, 1 or 0x10000 by the sign bit, is the pattern's sign spread over
// its half (one packed shift for both patterns of a word) plus 1.
RLK_DEV uint32_t window_bits(uint32_t w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 t = __builtin_bit_cast(u16x2, w) + u16x2{0x2000, 0x2000};
  return __builtin_bit_cast(uint32_t, t);
}

RLK_DEV void count8(uint32_t* hist, uint32_t* special, const uint4& q) {
  const uint32_t t = window_bits(q.x) & window_bits(q.y) & window_bits(q.z) & window_bits(q.w);
  if ((t & 0x40004000u) == 0x40004000u) {
    char* base = reinterpret_cast<char*>(hist);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    typedef short i16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // both patterns' signs at once: 0 or 0xffff per half
      const uint32_t sg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w[k]) >> 15);
      atomicAdd(reinterpret_cast<uint32_t*>(base + ((w[k] & 0x3fffu) << 2)), (sg & 0xffffu) + 1u);
      atomicAdd(reinterpret_cast<uint32_t*>(base + (((w[k] >> 16) & 0x3fffu) << 2)), (sg >> 16) + 1u);
    }
  } else {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      count_code(hist, special, w[k] & 0xffffu);
      count_code(hist, special, w[k] >> 16);
    }
  }
}

// Count of the value with merged key `key` (key = code | 0x8000 for a positive
// pattern, ~code & 0xffff for a negative one, 0x8000 for +-0), and the value.
RLK_DEV uint32_t key_count(const uint32_t* hist, int key, float* value, uint32_t n_zero) {
  if (key == 0x8000) {
    *value = 0.f;
    return n_zero;
  }
  if (key > 0x8000) {
    const int mag = key - 0x8000;
    *value = bf16_to_f32(uint16_t(mag));
    return (mag >= kMagLo && mag < kMagHi) ? (hist[widx(mag)] & 0xffffu) : 0u;
  }
  const int mag = 0x7fff - key;
  *value = bf16_to_f32(uint16_t(0x8000 | mag));
  return (mag >= kMagLo && mag < kMagHi) ? (hist[widx(mag)] >> 16) : 0u;
}

RLK_DEV uint32_t bf16_key_merged(uint16_t code) {
  if (code == 0x8000u) code = 0;
  return (code & 0x8000u) ? ((~uint32_t(code)) & 0xffffu) : (uint32_t(code) | 0x8000u);
}

RLK_DEV float merged_key_value(uint32_t key) {
  if (key == 0x8000u) return 0.f;
  return key > 0x8000u ? bf16_to_f32(uint16_t(key - 0x8000u)) : bf16_to_f32(uint16_t(~key & 0xffffu));
}

// exp((v - m) / T) for a bf16 value v and the row max m, in fp32. dv = v - m
// is exact (two bf16 values). With c = log2(e)/T split as c_hi + c_lo, the
// exponent x = dv*c is rounded to x_hi = fl(dv*c_hi) and its residual
// r = (dv*c_hi - x_hi) + dv*c_lo is recovered by an fma, so
// 2^x = 2^x_hi * (1 + r ln 2) carries ~1 ulp of error whatever |x| is.
struct MassScale {
  float c_hi, c_lo;
};

RLK_DEV MassScale mass_scale(double invT) {
  const double c = 1.4426950408889634 * invT;
  MassScale k;
  k.c_hi = float(c);
  k.c_lo = float(c - double(k.c_hi));
  return k;
}

// The hardware exp2 is used as is: below 2^-126 a mass is far under the
// resolution of the fp64 sums it enters (each row's max contributes 1).
RLK_DEV float code_mass(float dv, MassScale k) {
  const float xh = dv * k.c_hi;
  const float r = fmaf(dv, k.c_hi, -xh) + dv * k.c_lo;
  const float e = __builtin_amdgcn_exp2f(xh);
  return fmaf(e, r * 0.69314718f, e);
}

// ---------------------------------------------------------------------------
// Finisher group: waves kStreamWaves..15 post-process one row while the other
// waves stream the next. They synchronise among themselves through an LDS
// counter: every finisher wave runs the same uniform sequence of syncs, and
// all of them are resident in the block, so each wait ends.
// ---------------------------------------------------------------------------
constexpr int kMaxFW = kHT / kWave;              // every wave finishes the block's last row
struct FinScratch {
  int i[8][kMaxFW];
  uint64_t d[7][kMaxFW];   // fixed-point partial sums
  uint64_t bd[3];
  int bi[2];
  unsigned int bar;
  unsigned int handed_on;   // nonzero once any row of the block is handed on
};

template <int FW>
RLK_DEV void fsync(unsigned int* bar, unsigned int& epoch) {
  if constexpr (FW == kHT / kWave) {   // the whole block: the hardware barrier
    __syncthreads();
    return;
  }
  epoch += FW;
  if ((threadIdx.x & (kWave - 1)) == 0)
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < epoch)
    __builtin_amdgcn_s_sleep(1);
}

// The finisher's sums are exact: masses (and mass times d) enter them as
// unsigned fixed-point integers in units of 2^-kFxBits, so integer addition
// makes every total independent of how the terms are split across threads
// and waves. That keeps a row's outputs bitwise the same whether 4 waves
// finish it (while the others stream) or all 16 do (a block's last row),
// i.e. independent of the number of rows and of which rows share a block.
// A value below the unit is truncated; a row holds at most 2^24 values of
// mass <= 1 each, so 2^24 2^38 < 2^63 never overflows, and the truncation
// costs at most 2^-38 per term (Z >= 1: the max contributes 1).
constexpr int kFxBits = 38;
RLK_DEV uint64_t to_fx(double x) { return uint64_t(x * 0x1p38); }   // x in [0, 2^24)
RLK_DEV double from_fx(uint64_t u) { return double(u) * 0x1p-38; }

// Everything after counting, for one row: checksum and occupied range, max,
// Z and entropy, the top-p walk, outputs (or the hand-off flag), and zeroing
// the counters it used so the buffer is ready for the row after next.
template <int FW>
RLK_DEV void finish_row(const RowArgs& a, int64_t row, uint32_t* hist, uint32_t* special,
                        FinScratch& fs, unsigned int& epoch) {
  constexpr int FT = FW * kWave;                  // finisher threads: the last FT of the block
  int ft = int(threadIdx.x) - (kHT - FT);          // 0 .. FT-1
  // an opaque copy per row: otherwise the compiler hoists every per-thread
  // counter address and magnitude out of the row loop into registers
  asm volatile("" : "+v"(ft));
  const int lane = ft & (kWave - 1), fw = ft / kWave;
  const int64_t V = a.vocab;
  const uint16_t* rowp = reinterpret_cast<const uint16_t*>(a.logits) + row * a.row_stride;
  const int64_t y = a.targets[row];
  const bool y_ok = y >= 0 && y < V;
  const uint16_t cy = (ft == 0 && y_ok) ? rowp[y] : uint16_t(0);
  const float T = a.t_row ? a.t_row[row] : a.temperature;
  const float p = a.p_row ? a.p_row[row] : a.top_p;
  const int n_zero = int(special[0]), n_neginf = int(special[1]), n_other = int(special[2]);

  // ---- one sweep over the counters in 16-byte groups (4 magnitudes), a
  //      batch of reads in flight, with a few operations per group (this
  //      wave shares its SIMD's issue with three streaming waves): occupied
  //      range, and the groups holding the largest positive and the
  //      smallest negative magnitude ----
  {
    constexpr int kPer = kHWords / 4 / FT;            // groups per finisher thread
    constexpr int kBatch = kPer < 8 ? kPer : 8;
    // group q = ft + k*FT covers counters 4q..4q+3; counters below 0x2000
    // hold magnitudes 0x4000 above their index (the window's rotation), and
    // 0x2000 is a multiple of 4*FT, so the shift depends on k alone
    static_assert(0x2000 % (4 * FT) == 0, "rotation boundary on a k boundary");
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
    int tmin = 0x7fff, tmax = -1, pg = -1, ng_ = 0x8000;
#pragma unroll
    for (int k0 = 0; k0 < kPer; k0 += kBatch) {
      uint4 x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) x[u] = h4[ft + (k0 + u) * FT];
      __builtin_amdgcn_sched_barrier(0);   // every read issued before the first use
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int k = k0 + u;
        const int m0 = 4 * ft + 4 * k * FT + (4 * k * FT < 0x2000 ? 0x4000 : 0);
        const uint32_t o = x[u].x | x[u].y | x[u].z | x[u].w;
        tmin = min(tmin, o ? m0 : 0x7fff);
        tmax = max(tmax, o ? m0 + 3 : -1);
        pg = max(pg, (o & 0xffffu) ? m0 : -1);
        ng_ = min(ng_, (o >> 16) ? m0 : 0x8000);
      }
    }
    // the exact magnitudes inside this thread's two groups
    int pmax = -1, nmin = 0x8000;
    {
      const uint4 xp = h4[widx(pg >= 0 ? pg : 0x4000) >> 2];
      const uint4 xn = h4[widx(ng_ < 0x8000 ? ng_ : 0x4000) >> 2];
      if (pg >= 0)
        pmax = pg + ((xp.w & 0xffffu) ? 3 : (xp.z & 0xffffu) ? 2 : (xp.y & 0xffffu) ? 1 : 0);
      if (ng_ < 0x8000)
        nmin = ng_ + ((xn.x >> 16) ? 0 : (xn.y >> 16) ? 1 : (xn.z >> 16) ? 2 : 3);
    }
    const int mn_w = wave_min_i32(tmin), mx_w = wave_max_i32(tmax);
    const int pm_w = wave_max_i32(pmax), nm_w = wave_min_i32(nmin);
    if (lane == 0) {
      fs.i[1][fw] = mn_w;
      fs.i[2][fw] = mx_w;
      fs.i[3][fw] = pm_w;
      fs.i[4][fw] = nm_w;
    }
  }
  fsync<FW>(&fs.bar, epoch);
  const int wmin = wave_min_i32(lane < FW ? fs.i[1][lane] : 0x7fff);
  const int wmax = wave_max_i32(lane < FW ? fs.i[2][lane] : -1);
  const int maxpos = wave_max_i32(lane < FW ? fs.i[3][lane] : -1);
  const int minneg = wave_min_i32(lane < FW ? fs.i[4][lane] : 0x8000);
  // the occupied range as 4-aligned groups of magnitudes: group g holds
  // magnitudes g0 + 4g .. g0 + 4g + 3, one 16-byte read (the rotation keeps
  // such a group contiguous)
  const int g0 = wmin & ~3;
  const int ng = ((wmax | 3) - g0 + 1) >> 2;   // <= 0 when nothing was counted

  // largest value: highest magnitude with a positive pattern; else zero;
  // else the negative pattern of smallest magnitude
  float mval;
  int kmax;
  if (maxpos >= 0) {
    mval = bf16_to_f32(uint16_t(maxpos));
    kmax = 0x8000 + maxpos;
  } else if (n_zero > 0) {
    mval = 0.f;
    kmax = 0x8000;
  } else {
    mval = bf16_to_f32(uint16_t(0x8000 | minneg));
    kmax = 0x7fff - minneg;
  }
  const double invT = 1.0 / double(T);
  const float invTf = float(invT);
  const MassScale ks = mass_scale(invT);

  // ---- over the occupied groups, 2 in flight (more would spill): the
  //      checksum of all counts, and Z and -sum e*d over the distinct
  //      values (formed for every row; used only when the row is live): a
  //      16-byte group's 8 terms summed in fp64 in a fixed order, the group
  //      sum converted to fixed point ----
  {
    uint32_t t_acc = 0;
    uint64_t zt = 0, st = 0;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
    for (int gb = 0; gb < ng; gb += 2 * FT) {
      uint4 x[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int g = gb + ft + u * FT;
        x[u] = g < ng ? h4[widx(g0 + 4 * g) >> 2] : make_uint4(0u, 0u, 0u, 0u);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m0 = g0 + 4 * (gb + ft + u * FT);
        const uint32_t c[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        double zg = 0.0, sg = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          t_acc = __builtin_amdgcn_sad_u16(c[j], 0u, t_acc);
          const float v = __uint_as_float(uint32_t(m0 + j) << 16);   // the positive value
#pragma unroll
          for (int sgn = 0; sgn < 2; ++sgn) {
            const uint32_t n = sgn ? (c[j] >> 16) : (c[j] & 0xffffu);
            // v - max, clamped to <= 0: a value above the max is absent from
            // the row (n = 0), and the clamp keeps its mass finite so that it
            // contributes exactly 0; present values are unchanged
            const float dv = fminf((sgn ? -v : v) - mval, 0.f);
            const float e = code_mass(dv, ks) * float(n);
            zg += double(e);
            sg -= double(e) * double(dv * invTf);
          }
        }
        zt += to_fx(zg);
        st += to_fx(sg);
        __builtin_amdgcn_sched_barrier(0);   // one group's arithmetic at a time
      }
    }
    if (ft == 0 && n_zero > 0) {   // the +-0 group
      const float dv = -mval;
      const float e = code_mass(dv, ks) * float(n_zero);
      zt += to_fx(double(e));
      st += to_fx(-(double(e) * double(dv * invTf)));
    }
    const int t_w = wave_total(int(t_acc));
    zt = wave_total(zt);
    st = wave_total(st);
    if (lane == 0) {
      fs.i[0][fw] = t_w;
      fs.d[0][fw] = zt;
      fs.d[1][fw] = st;
    }
  }
  fsync<FW>(&fs.bar, epoch);
  const int tot = fold_partials(fs.i[0], FW);

  uint8_t flags = 0;
  if (!y_ok) flags |= kBadTarget;
  if (!param_ok(T, p) || row_top_k(a, row) < 0) flags |= kBadParam;
  if (n_zero == 0 && n_neginf == int(V)) flags |= kNonFinite;
  // a value held > 65535 times wraps its counter; +inf, NaN and extreme
  // magnitudes are not counted: the generic kernel redoes such rows
  const bool handoff = n_other != 0 || tot + n_zero + n_neginf != int(V);
  const bool live = !handoff && !(flags & (kBadParam | kNonFinite));
  if (ft == 0) {
    a.fallback[row] = handoff ? 1 : 0;
    if (handoff) fs.handed_on = 1u;
    if (!handoff && !live) store_nan_row(a, row, flags);
  }

  if (live) {
    const uint64_t Zu = fold_partials(fs.d[0], FW);
    const uint64_t Su = fold_partials(fs.d[1], FW);
    const double Z = from_fx(Zu);
    const double S = -from_fx(Su);

    // ---- top-k: the floor's merged key; the cut below stops there ----
    const float floor_v = row_floor(a, row);
    const bool has_floor = floor_v > -INFINITY;
    const int lo_key =
        has_floor ? int(bf16_key_merged(uint16_t(__float_as_uint(floor_v) >> 16))) : kKeyLo;
    // the mass at or above the floor (the top-k set), from the same per-key
    // terms as the walk below, so that the walk's sums reach it exactly
    double Zf = Z;
    if (has_floor && p < 1.f) {
      uint64_t zf = 0;
      for (int key = kmax - ft; key >= lo_key; key -= FT) {
        float v;
        const int n = int(key_count(hist, key, &v, uint32_t(n_zero)));
        if (n) zf += to_fx(double(code_mass(v - mval, ks) * float(n)));
      }
      zf = wave_total(zf);
      if (lane == 0) fs.d[6][fw] = zf;
      fsync<FW>(&fs.bar, epoch);
      Zf = from_fx(fold_partials(fs.d[6], FW));
    }

    // ---- top-p cut: walk merged keys down from the max, FT at a time; the
    //      masses per key in fixed point, so every cumulative sum is exact.
    //      With top-k at top-p 1 nothing crosses and the walk keeps every
    //      value down to the floor ----
    double Zs = Z, Ss = S, Mgt = 0.0;
    uint32_t tau_key = 0;
    int size = int(V) - n_neginf;
    const bool cut = p < 1.f || has_floor;
    if (cut) {
      const double thr = p < 1.f ? double(p) * Zf : INFINITY;
      uint64_t cz = 0, cs = 0;
      int cn = 0;
      bool found = false;
      int par = 0;
      for (int k0 = kmax; !found && k0 >= lo_key; k0 -= FT, par ^= 1) {
        const int key = k0 - ft;
        uint64_t mass = 0, ms = 0;
        int n = 0;
        if (key >= lo_key) {
          float v;
          n = int(key_count(hist, key, &v, uint32_t(n_zero)));
          if (n) {
            const float dv = v - mval;
            const float e = code_mass(dv, ks) * float(n);
            mass = to_fx(double(e));
            ms = to_fx(-(double(e) * double(dv * invTf)));
          }
        }
        const uint64_t iz = wave_scan_incl(mass), is = wave_scan_incl(ms);
        const int in = wave_scan_incl(n);
        if (lane == kWave - 1) {
          fs.d[2 + 2 * par][fw] = iz;
          fs.d[3 + 2 * par][fw] = is;
          fs.i[5 + par][fw] = in;
        }
        fsync<FW>(&fs.bar, epoch);
        // wave partials in lanes 0..FW-1: exclusive prefixes; the inclusive
        // cumulative mass of a key, compared with p Z as a double (the
        // conversion of an exact integer: the same whoever forms it)
        const uint64_t pz = lane < FW ? fs.d[2 + 2 * par][lane] : uint64_t(0);
        const uint64_t ps = lane < FW ? fs.d[3 + 2 * par][lane] : uint64_t(0);
        const int pn = lane < FW ? fs.i[5 + par][lane] : 0;
        const uint64_t ez = wave_shift_up(wave_scan_incl(pz));
        const uint64_t es = wave_shift_up(wave_scan_incl(ps));
        const int en = wave_shift_up(wave_scan_incl(pn));
        const uint64_t wcross = __ballot(lane < FW && from_fx(cz + ez + pz) >= thr);
        const int cross_wave = wcross ? __ffsll((unsigned long long)wcross) - 1 : -1;
        if (cross_wave >= 0) {
          if (fw == cross_wave) {
            const uint64_t wbz = readlane_u64(ez, cross_wave);
            const uint64_t wbs = readlane_u64(es, cross_wave);
            const int wbn = int(readlane_u32(uint32_t(en), cross_wave));
            const uint64_t incl = cz + wbz + iz;
            const uint64_t bal = __ballot(from_fx(incl) >= thr);
            const int first = __ffsll((unsigned long long)bal) - 1;
            if (lane == first) {
              fs.bd[0] = incl;
              fs.bd[1] = cs + wbs + is;
              fs.bd[2] = incl - mass;
              fs.bi[0] = key;
              fs.bi[1] = cn + wbn + in;
            }
          }
          fsync<FW>(&fs.bar, epoch);
          Zs = from_fx(fs.bd[0]);
          Ss = -from_fx(fs.bd[1]);
          Mgt = from_fx(fs.bd[2]);
          tau_key = uint32_t(fs.bi[0]);
          size = fs.bi[1];
          found = true;
        } else {
          cz += readlane_u64(ez, FW - 1) + readlane_u64(pz, FW - 1);
          cs += readlane_u64(es, FW - 1) + readlane_u64(ps, FW - 1);
          cn += int(readlane_u32(uint32_t(en), FW - 1)) + int(readlane_u32(uint32_t(pn), FW - 1));
        }
      }
      if (!found) {   // top-p 1 with top-k, or truncation left the mass just
                      // short of p: keep every value down to the floor
        Zs = from_fx(cz);
        Ss = -from_fx(cs);
        Mgt = Zs;
        tau_key = uint32_t(lo_key);
        size = cn;
      }
    }

    // the two logarithms and quotients on lanes 0 and 1 of the first
    // finisher wave at once, then the outputs from its lane 0
    double logZ = 0.0, logZs = 0.0, eZ = 0.0, eZs = 0.0;
    if (fw == 0) {
      const bool second = lane == 1;
      const double lg = log(second ? Zs : Z);
      const double q = (second ? Ss : S) / (second ? Zs : Z);
      logZ = readlane_f64(lg, 0);
      logZs = readlane_f64(lg, 1);
      eZ = readlane_f64(q, 0);
      eZs = readlane_f64(q, 1);
    }
    if (ft == 0) {
      const float h_full = float(logZ - eZ);
      const float h_trunc = float(logZs - eZs);
      float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
      if (y_ok) {
        const float vy = bf16_to_f32(cy);
        if (vy == -INFINITY) {
          lpf = -INFINITY;
          lpt = -INFINITY;
          flags |= kOutside;
        } else {
          lpf = token_logprob(vy, double(mval), invT, logZ);
          if (!cut || bf16_key_merged(cy) >= tau_key) {
            lpt = token_logprob(vy, double(mval), invT, logZs);
          } else {
            lpt = -INFINITY;
            flags |= kOutside;
          }
        }
      }
      float tau = -INFINITY;
      if (cut) {
        tau = merged_key_value(tau_key);
        const double pp = double(p);
        if (p < 1.f && (fabs(Mgt / Zf - pp) <= kBoundaryEps || fabs(Zs / Zf - pp) <= kBoundaryEps))
          flags |= kBoundary;
      }
      const double mT = double(mval) * invT;
      if (a.score_stats) {
        a.score_stats[2 * row] = double(mval);
        a.score_stats[2 * row + 1] = logZs;
      }
      store_row(a, row, lpf, lpt, h_full, h_trunc, size, tau, flags, float(mT + logZs),
                float(mT + eZs));
    }
  }

  // ---- release the buffer: every nonzero counter lies in [wmin, wmax] ----
  {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (int g = ft; g < ng; g += FT) h4[widx(g0 + 4 * g) >> 2] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (ft == 0) special[0] = special[1] = special[2] = 0;
}

// 16 bytes of a row read once: a non-temporal load, so the stream does not
// displace reusable lines in the caches.
RLK_DEV uint4 stream_load(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Stream one row into a counter buffer with threads 0..NS-1 of the block.
template <bool kVec, int NS>
RLK_DEV void stream_row(const RowArgs& a, int64_t row, int64_t nvec, uint32_t* h, uint32_t* sp) {
  const int tid = threadIdx.x;
  const int64_t V = a.vocab;
  const uint16_t* rowp = reinterpret_cast<const uint16_t*>(a.logits) + row * a.row_stride;
  if (kVec) {
    const uint4* v4 = reinterpret_cast<const uint4*>(rowp);
    int64_t i = tid;
    for (; i + (kUnroll - 1) * NS < nvec; i += kUnroll * NS) {
      uint4 q[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) q[u] = stream_load(v4 + i + u * NS);
      // all kUnroll loads issued before the first is used (the scheduler
      // would otherwise wait for the first before issuing the rest)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) count8(h, sp, q[u]);
    }
    for (; i < nvec; i += NS) count8(h, sp, stream_load(v4 + i));
    for (int64_t j = (nvec << 3) + tid; j < V; j += NS) count_code(h, sp, rowp[j]);
  } else {
    for (int64_t j = tid; j < V; j += NS) count_code(h, sp, rowp[j]);
  }
}

// One persistent block per CU; block b takes rows b, b + G, b + 2G, ...
// (G = gridDim.x). Step s: waves 0..kStreamWaves-1 stream row R_s into
// counter buffer s & 1 while (from step 1 on) the finisher waves
// post-process row R_{s-1} from the other buffer, one block barrier between
// steps; the last row is post-processed by all 16 waves.
// Rows the finishers hand on (see finish_row) are then redone by the whole
// block with the generic algorithm, in the same launch.
template <bool kVec>
__global__ __launch_bounds__(kHT) void bf16_hist_rows(RowArgs a) {
  __shared__ uint32_t hist[2][kHWords];
  __shared__ uint32_t special[2][4];
  __shared__ FinScratch fs;
  static_assert(sizeof(GenScratch) <= sizeof(hist), "generic scratch reuses the counters");

  const int tid = threadIdx.x, wid = tid / kWave;
  const int64_t V = a.vocab;
  const int64_t nvec = kVec ? (V >> 3) : 0;
  const int64_t N = a.n_rows;
  const int64_t G = gridDim.x;

  {
    uint4* h4 = reinterpret_cast<uint4*>(&hist[0][0]);
    for (int i = tid; i < 2 * kHWords / 4; i += kHT) h4[i] = make_uint4(0, 0, 0, 0);
  }
  if (tid < 8) special[tid >> 2][tid & 3] = 0;
  if (tid == 0) {
    fs.bar = 0;
    fs.handed_on = 0;
  }
  unsigned int epoch = 0;
  __syncthreads();

  int64_t prev = blockIdx.x;   // the row in the buffer the finishers read next
  // the first row by the streaming waves alone (all 16 waves measured slower)
  if (prev < N && wid < kStreamWaves) stream_row<kVec, kStreamers>(a, prev, nvec, hist[0], special[0]);
  __syncthreads();
  int s = 1;
  for (int64_t cur = prev + G; cur < N; cur += G, ++s) {
    const int b = s & 1;
    if (wid < kStreamWaves) {
      // one copy per buffer, so that its LDS base is a constant
      if (b)
        stream_row<kVec, kStreamers>(a, cur, nvec, hist[1], special[1]);
      else
        stream_row<kVec, kStreamers>(a, cur, nvec, hist[0], special[0]);
    } else {
      finish_row<kFW>(a, prev, hist[b ^ 1], special[b ^ 1], fs, epoch);
    }
    __syncthreads();
    prev = cur;
  }
  if (prev < N) {   // the last row: every wave finishes it
    epoch = __hip_atomic_load(&fs.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    finish_row<kMaxFW>(a, prev, hist[(s & 1) ^ 1], special[(s & 1) ^ 1], fs, epoch);
    __syncthreads();
  }
  // rows handed on by this block's finishers (flags written before the last
  // barrier), redone with the counters' LDS as scratch; the block-local mark
  // skips the scan of the flags (one dependent global read per row) in the
  // normal case, where none was handed on
  if (fs.handed_on == 0u) return;
  GenScratch& gs = *reinterpret_cast<GenScratch*>(&hist[0][0]);
  for (int64_t row = blockIdx.x; row < N; row += gridDim.x) {
    if (a.fallback[row]) {
      generic_row<uint16_t, kHT>(a, row, gs);
      __syncthreads();
    }
  }
}

// ===========================================================================
// fp32 rows: three streaming passes with float4 loads (one 512-thread block
// per row). Pass 1: max and finite count. Pass 2: Z, sum e d and a histogram
// of fixed-point masses over bins of equal width in d = (z - max)/T (64 bins
// per nat; a bin index never increases with z, so every bin above the
// crossing bin holds only larger values). Pass 3: the truncated sums of the
// bins above the crossing bin, and the keys of the crossing bin's elements
// collected in LDS; sorted there, they give the exact threshold. A row whose
// crossing bin holds more than kCand elements is redone by the generic
// algorithm in the same block.
// ===========================================================================
// threads per block: 512, so that two blocks share a CU (66 KB of LDS and at
// most 128 VGPRs each) and one row's barrier-bound phases (the bin walk, the
// sort of the crossing bin, the block reductions) overlap the other row's
// streaming passes; a 1024-thread block held its CU alone
constexpr int kF32T = 512;
constexpr int kF32WavesPerSimd = 4;   // two blocks of 8 waves per CU
constexpr int kFBins = 4096;          // bins of d: [b / 64, (b + 1) / 64) nats below the max
constexpr float kFBinPerNat = 64.f;
constexpr int kCand = 8192;           // crossing-bin elements resolved in LDS

template <int NT>
RLK_DEV int walk_bins(const uint64_t* bins, int nbins, uint64_t thr, uint64_t* above,
                      uint64_t* su64, int* si, uint64_t* bslot) {
  uint64_t carry = 0;
  for (int base = 0; base < nbins; base += NT) {
    const int b = base + int(threadIdx.x);
    const uint64_t v = b < nbins ? bins[b] : 0ull;
    uint64_t tot;
    const uint64_t incl = block_inclusive_scan(v, su64, &tot);
    const int cand = (v != 0ull && carry + incl >= thr) ? int(threadIdx.x) : NT;
    const int first = block_min(cand, si);
    if (first < NT) {
      if (int(threadIdx.x) == first) *bslot = carry + incl - v;
      __syncthreads();
      *above = *bslot;
      __syncthreads();
      return base + first;
    }
    carry += tot;
  }
  *above = carry;
  return -1;
}

// Per-row constants of the fp32 kernel.
struct F32Scale {
  double c;      // log2(e) / T
  double mc;     // m c, m the row max
  double binc;   // -(bins per nat) ln 2: the bin of x is floor(x binc)
};

// x = (z - m) log2(e) / T in fp64: one fma of z c - m c, monotone in z.
RLK_DEV double f32_x(float z, const F32Scale& k) { return fma(double(z), k.c, -k.mc); }

// exp((z - m)/T) = 2^x in fp32 to about 1 ulp: x rounded to fp32 x_hi for the
// hardware exp2 and its residual restored to first order, 2^x = 2^x_hi (1 +
// (x - x_hi) ln 2) (|x - x_hi| <= 2^-18 wherever the mass is above 2^-64).
// Below 2^-126 a mass is far under the fixed-point unit and the sums'
// resolution, whatever the denormal handling.
RLK_DEV float f32_mass(double x) {
  const float xh = float(x);
  const float r = float(x - double(xh));
  const float e = __builtin_amdgcn_exp2f(xh);
  return fmaf(e, r * 0.69314718f, e);
}

// The d bin of x (64 bins per nat below the max, the last one open-ended): a
// bin index never increases with z.
RLK_DEV int f32_bin(double x, const F32Scale& k) {
  const double u = x * k.binc;
  return u < double(kFBins - 1) ? int(u) : kFBins - 1;
}

// round(e * 2^39) for e in [0, 1], ties to even: e 2^39 is exact, and adding
// 2^52 in fp64 leaves the integer in the low bits of the significand.
RLK_DEV uint64_t f32_fixed(double e) {
#pragma clang fp contract(off)   // a multiply and an add: an fma costs two moves per element
  const double v = e * 549755813888.0 + 4503599627370496.0;
  return uint64_t(__double_as_longlong(v)) - 0x4330000000000000ull;
}
constexpr double kFixUnit = 1.0 / 549755813888.0;   // 2^-39

// Visit every element of a row, 16 bytes per lane per load with kF32Unroll
// loads in flight per thread (the loads of a group are issued before any of
// them is used).
constexpr int kF32Unroll = 4;
template <bool kVec, typename F>
RLK_DEV void for_each_f32(const float* rowp, int64_t V, F&& f) {
  if (kVec) {
    const int64_t V4 = V >> 2;
    const float4* p4 = reinterpret_cast<const float4*>(rowp);
    int64_t i = threadIdx.x;
    for (; i + (kF32Unroll - 1) * kF32T < V4; i += kF32Unroll * kF32T) {
      float4 q[kF32Unroll];
#pragma unroll
      for (int u = 0; u < kF32Unroll; ++u) q[u] = p4[i + u * kF32T];
      __builtin_amdgcn_sched_barrier(0);   // all loads issued before the first use
#pragma unroll
      for (int u = 0; u < kF32Unroll; ++u) {
        const int64_t e = 4 * (i + u * kF32T);
        f(q[u].x, e);
        f(q[u].y, e + 1);
        f(q[u].z, e + 2);
        f(q[u].w, e + 3);
      }
    }
    for (; i < V4; i += kF32T) {
      const float4 v = p4[i];
      f(v.x, 4 * i);
      f(v.y, 4 * i + 1);
      f(v.z, 4 * i + 2);
      f(v.w, 4 * i + 3);
    }
    for (int64_t j = 4 * V4 + threadIdx.x; j < V; j += kF32T) f(rowp[j], j);
  } else {
    for (int64_t i = threadIdx.x; i < V; i += kF32T) f(rowp[i], i);
  }
}

template <bool kVec>
__global__ __launch_bounds__(kF32T, kF32WavesPerSimd) void f32_rows(RowArgs a) {
  __shared__ union {
    struct {
      uint64_t hist[kFBins];
      uint32_t cand[kCand];
    } f;
    GenScratch g;
  } sm;
  uint64_t* hist = sm.f.hist;
  uint32_t* cand = sm.f.cand;
  __shared__ double sd[kF32T / kWave];
  __shared__ uint64_t su64[kF32T / kWave];
  __shared__ int si[kF32T / kWave];
  __shared__ float sf[kF32T / kWave];
  __shared__ uint64_t bslot;
  __shared__ unsigned int ncand_s;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t V = a.vocab;
  const float* rowp = reinterpret_cast<const float*>(a.logits) + row * a.row_stride;

  // the producer's per-row max (order key) and non-finite flag, cleared for
  // the producer's next block of rows
  bool known = false;
  float known_max = 0.f;
  if (a.zmax_key) {
    const uint32_t k = a.zmax_key[row], zb = a.zbad[row];
    __syncthreads();
    if (tid == 0) {
      a.zmax_key[row] = 0u;
      a.zbad[row] = 0u;
    }
    if (zb == 0u && k != 0u) {
      known = true;
      known_max = key_f32(k);
    }
  }
  const float Tv = a.t_row ? a.t_row[row] : a.temperature;
  const float p = a.p_row ? a.p_row[row] : a.top_p;
  const int64_t y = a.targets[row];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  if (!param_ok(Tv, p) || row_top_k(a, row) < 0) {
    if (tid == 0) store_nan_row(a, row, flags | kBadParam);
    return;
  }
  // top-k: only values >= the floor take part in the cut
  const float floor_v = row_floor(a, row);
  const bool has_floor = floor_v > -INFINITY;
  const uint32_t fk = has_floor ? f32_key(floor_v) : 0u;

  // ---- pass 1: max, finite count, non-finite detection (or the producer's
  // max when it saw only finite logits) ----
  float mx = -INFINITY;
  int bad = 0;
  uint32_t nfin = 0;
  if (known) {
    mx = known_max;
    nfin = uint32_t(V);
  } else {
    for_each_f32<kVec>(rowp, V, [&](float z, int64_t) {
      if (z != z || z == INFINITY) bad = 1;
      else if (z > -INFINITY) {
        mx = fmaxf(mx, z);
        ++nfin;
      }
    });
    mx = block_max(mx, sf);
    bad = block_max(bad, si);
    nfin = uint32_t(block_sum(uint64_t(nfin), su64));
  }
  if (bad || nfin == 0) {
    if (tid == 0) store_nan_row(a, row, flags | kNonFinite);
    return;
  }
  const double m = double(mx);
  const double invT = 1.0 / double(Tv);
  F32Scale ks;
  ks.c = 1.4426950408889634 * invT;
  ks.mc = m * ks.c;
  ks.binc = -double(kFBinPerNat) * 0.6931471805599453;
  // every element below this has zero mass at fp32 precision; clamping -inf
  // to it keeps the arithmetic free of inf - inf
  const float zfloor = float(m - 1e30);
  const bool cut_p = p < 1.f;
  const bool cut = cut_p || has_floor;
  // sum e d over the row is needed for the full entropy (when the caller
  // asks for it) and at top-p 1 for the truncated one too
  const bool need_s = a.ent_full != nullptr || !cut_p;

  // ---- pass 2: Z (fixed point), sum e d, histogram of fixed-point masses
  //      over d bins (with top-k, of the values at or above its floor only) ----
  if (cut_p) {
    for (int i = tid; i < kFBins; i += kF32T) hist[i] = 0ull;
    if (tid == 0) ncand_s = 0;
    __syncthreads();
  }
  // Per element without branches except the atomic; the top-p histogram,
  // the top-k floor and the entropy sum are compile-time variants.
  // (wt: the cut's mass, at or above the top-k floor; wall: the whole row's,
  // kept apart only when a floor makes the two differ)
  double st = 0.0;
  uint64_t wt = 0, wall = 0;
  auto pass2 = [&](auto with_hist, auto with_floor, auto with_s) {
    for_each_f32<kVec>(rowp, V, [&](float z, int64_t) {
      const double x = f32_x(fmaxf(z, zfloor), ks);
      const double ed = double(f32_mass(x));
      const uint64_t w = f32_fixed(ed);
      if constexpr (decltype(with_s)::value) st = fma(ed, x * 0.6931471805599453, st);
      if constexpr (decltype(with_hist)::value) {
        uint64_t wk = w;
        if constexpr (decltype(with_floor)::value) {
          wall += w;
          wk = f32_key(z) >= fk ? w : 0ull;
        }
        wt += wk;
        if (wk)
          atomicAdd(reinterpret_cast<unsigned long long*>(&hist[f32_bin(x, ks)]),
                    (unsigned long long)wk);
      } else {
        wt += w;
      }
    });
  };
  constexpr std::true_type Y{};
  constexpr std::false_type N{};
  if (!cut_p) {
    pass2(N, N, Y);
  } else if (has_floor) {
    pass2(Y, Y, N);
    if (need_s)   // the full entropy with top-k and top-p: a pass of its own
      for_each_f32<kVec>(rowp, V, [&](float z, int64_t) {   // (one loop would spill)
        const double x = f32_x(fmaxf(z, zfloor), ks);
        st = fma(double(f32_mass(x)), x * 0.6931471805599453, st);
      });
  } else {
    need_s ? pass2(Y, N, Y) : pass2(Y, N, N);
  }
  const uint64_t wt_sum = cut_p ? block_sum(wt, su64) : 0ull;
  const uint64_t wall_sum = (cut_p && !has_floor) ? wt_sum : block_sum(cut_p ? wall : wt, su64);
  const double Z = double(wall_sum) * kFixUnit;
  const double S = need_s ? block_sum(st, sd) : 0.0;

  double Zs = Z, Ss = S;
  uint32_t tau_key = 0;
  uint32_t size = nfin;
  if (!cut_p && has_floor) {   // top-k at top-p 1: S is the top-k set
    uint64_t zs = 0;
    double ss = 0.0;
    uint32_t cnt = 0;
    for_each_f32<kVec>(rowp, V, [&](float z, int64_t) {
      const bool in = z > -INFINITY && f32_key(z) >= fk;
      const double x = f32_x(fmaxf(z, zfloor), ks);
      const double ed = in ? double(f32_mass(x)) : 0.0;
      zs += f32_fixed(ed);
      ss = fma(ed, x * 0.6931471805599453, ss);
      cnt += in ? 1u : 0u;
    });
    Zs = double(block_sum(zs, su64)) * kFixUnit;
    Ss = block_sum(ss, sd);
    size = uint32_t(block_sum(uint64_t(cnt), su64));
    tau_key = fk;
  }
  if (cut_p) {
    const uint64_t W = wt_sum;
    const uint64_t thr = uint64_t(ceil(double(p) * double(W)));
    uint64_t above = 0;
    int bstar = walk_bins<kF32T>(hist, kFBins, thr, &above, su64, si, &bslot);
    if (bstar < 0) bstar = kFBins - 1;   // unreachable: the total mass reaches thr

    // ---- pass 3: sum e d above the crossing bin; its elements' keys to LDS
    // (Z_S itself is exact in fixed point: the mass above the crossing bin
    // plus the crossing bin's kept masses). The sum takes exp2 of the
    // fp32-rounded exponent: about 2^-24 |x| ln 2 relative per element, and
    // weighted by mass |x| averages at most log2 of the element count (x =
    // log2 of the element's mass relative to the max), so it is off by under
    // 2e-6 relative. The cut never uses it.
    double ss = 0.0;
    uint32_t cnt = 0;
    for_each_f32<kVec>(rowp, V, [&](float z, int64_t) {
      const double x = f32_x(fmaxf(z, zfloor), ks);
      const int b = z > -INFINITY ? f32_bin(x, ks) : kFBins;   // -inf: in no bin
      const bool in = b < bstar;
      const float xf = float(x);
      const float e = in ? __builtin_amdgcn_exp2f(xf) : 0.f;
      ss = fma(double(e), double(xf * 0.69314718f), ss);
      cnt += in ? 1u : 0u;
      if (b == bstar && f32_key(z) >= fk) {   // below the top-k floor: not a candidate
        const unsigned int slot = atomicAdd(&ncand_s, 1u);
        if (slot < unsigned(kCand)) cand[slot] = f32_key(z);
      }
    });
    __syncthreads();
    const int nc = int(ncand_s);
    if (nc > kCand) {   // too many elements in one bin: the generic algorithm resolves the row
      __syncthreads();
      generic_row<float, kF32T>(a, row, sm.g);
      return;
    }
    // sort the crossing bin's keys, descending (bitonic over a power of two)
    int n2 = 1;
    while (n2 < nc) n2 <<= 1;
    for (int i = nc + tid; i < n2; i += kF32T) cand[i] = 0u;
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kF32T) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t x = cand[i], w = cand[ixj];
            if (((i & k) == 0) ? (x < w) : (x > w)) {
              cand[i] = w;
              cand[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    // walk the sorted keys until the cumulative mass reaches thr
    uint64_t carry = above;
    int tau_idx = nc - 1;
    for (int base = 0; base < nc; base += kF32T) {
      const int i = base + tid;
      const uint64_t v = i < nc ? f32_fixed(double(f32_mass(f32_x(key_f32(cand[i]), ks)))) : 0ull;
      uint64_t tot;
      const uint64_t incl = block_inclusive_scan(v, su64, &tot);
      const int c = (i < nc && carry + incl >= thr) ? tid : kF32T;
      const int first = block_min(c, si);
      if (first < kF32T) {
        tau_idx = base + first;
        break;
      }
      carry += tot;
    }
    tau_key = cand[tau_idx];
    // truncated sums over the crossing bin's kept keys (key >= tau), in sorted order
    uint64_t mgt = 0, mat = 0;
    for (int i = tid; i < nc; i += kF32T) {
      const uint32_t k = cand[i];
      if (k < tau_key) continue;
      const double x = f32_x(key_f32(k), ks);
      const double ed = double(f32_mass(x));
      ss = fma(ed, x * 0.6931471805599453, ss);
      ++cnt;
      if (k > tau_key) mgt += f32_fixed(ed);
      else mat += f32_fixed(ed);
    }
    Ss = block_sum(ss, sd);
    size = uint32_t(block_sum(uint64_t(cnt), su64));
    mgt = above + block_sum(mgt, su64);
    mat = block_sum(mat, su64);
    Zs = double(mgt + mat) * kFixUnit;
    if (tid == 0) {
      const double pp = double(p);
      if (fabs(double(mgt) / double(W) - pp) <= kBoundaryEps ||
          fabs(double(mgt + mat) / double(W) - pp) <= kBoundaryEps)
        flags |= kBoundary;
    }
  }

  if (tid == 0) {
    const double logZ = log(Z), logZs = log(Zs);
    float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
    if (!(flags & kBadTarget)) {
      const float zy = rowp[y];
      if (!(zy > -INFINITY)) {
        lpf = -INFINITY;
        lpt = -INFINITY;
        flags |= kOutside;
      } else {
        lpf = token_logprob(zy, m, invT, logZ);
        if (!cut || f32_key(zy) >= tau_key) {
          lpt = token_logprob(zy, m, invT, logZs);
        } else {
          lpt = -INFINITY;
          flags |= kOutside;
        }
      }
    }
    const float tau = cut ? key_f32(tau_key) : -INFINITY;
    if (a.score_stats) {
      a.score_stats[2 * row] = m;
      a.score_stats[2 * row + 1] = logZs;
    }
    const float h_full = need_s ? float(logZ - S / Z) : __builtin_nanf("");
    store_row(a, row, lpf, lpt, h_full, float(logZs - Ss / Zs), int32_t(size), tau, flags,
              float(m * invT + logZs), float(m * invT + Ss / Zs));
  }
}


// ===========================================================================
// Top-k floor of each row (opt-in top-k): v_k, the k-th largest finite
// logit (ties counted one by one), by an exact radix select on the order
// keys, 8 bits per round: 4 rounds for fp32 logits, 2 for bf16 ones (their
// keys have 16 zero low bits). -inf when the row has no top-k (k = 0), when k
// is at least its number of finite values (the top-k set is then every
// finite value) or when k < 0 (the row kernel flags that row). NaN and +inf
// entries are not counted; such a row gets NaN outputs from the row kernel.
// ===========================================================================
constexpr int kKT = 256;   // one thread per 8-bit digit

template <typename T>
__global__ __launch_bounds__(kKT) void topk_floor_rows(RowArgs a, float* floor_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t su64[kKT / kWave];
  __shared__ int si[kKT / kWave];
  __shared__ int64_t above_s;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t V = a.vocab;
  const T* rowp = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;
  const int64_t k = row_top_k(a, row);
  if (k <= 0) {   // uniform across the block
    if (tid == 0) floor_out[row] = -INFINITY;
    return;
  }
  constexpr int kRounds = sizeof(T) == 2 ? 2 : 4;
  uint32_t prefix = 0;   // the key bits found so far
  int64_t need = k;      // rank still to find among the keys with that prefix
  for (int r = 0; r < kRounds; ++r) {
    const int shift = 24 - 8 * r;
    const uint32_t hi_mask = r == 0 ? 0u : (0xffffffffu << (shift + 8));
    hist[tid] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < V; i += kKT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY) || !(z < INFINITY)) continue;   // -inf, +inf, NaN
      const uint32_t key = f32_key(z);
      if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    // digits from the top: the first whose cumulative count reaches `need`
    const uint32_t c = hist[255 - tid];
    uint64_t tot;
    const uint64_t incl = block_inclusive_scan(uint64_t(c), su64, &tot);
    if (r == 0 && int64_t(tot) <= k) {   // k covers every finite value: no cut
      if (tid == 0) floor_out[row] = -INFINITY;
      return;
    }
    const int first = block_min((c != 0u && int64_t(incl) >= need) ? tid : kKT, si);
    if (tid == first) above_s = int64_t(incl) - int64_t(c);
    __syncthreads();
    need -= above_s;
    prefix |= uint32_t(255 - first) << shift;
    __syncthreads();
  }
  if (tid == 0) floor_out[row] = key_f32(prefix);
}

}  // namespace

// workspace: [0, n_rows) hand-off flags of the bf16 histogram path, then
// (256-byte aligned) each row's top-k floor, fp32 [n_rows]
size_t logits_rows_workspace(int64_t n_rows, int64_t vocab, int dtype) {
  (void)vocab;
  (void)dtype;
  return size_t((n_rows + 255) / 256 * 256) + size_t((4 * n_rows + 255) / 256 * 256);
}

hipError_t launch_logits_rows(const RowArgs& a, int dtype, void* workspace, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  RowArgs args = a;
  args.fallback = reinterpret_cast<uint8_t*>(workspace);
  const dim3 grid(unsigned(a.n_rows));
  if (a.top_k > 0 || a.k_row) {   // top-k: each row's floor first
    float* fl = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                         (a.n_rows + 255) / 256 * 256);
    if (dtype == 0)
      hipLaunchKernelGGL(topk_floor_rows<float>, grid, dim3(kKT), 0, stream, args, fl);
    else
      hipLaunchKernelGGL(topk_floor_rows<uint16_t>, grid, dim3(kKT), 0, stream, args, fl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    args.kfloor = fl;
  } else {
    args.kfloor = nullptr;
  }
  if (dtype == 0) {  // fp32
    const bool vec4 = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 4 == 0);
    if (vec4)
      hipLaunchKernelGGL(f32_rows<true>, grid, dim3(kF32T), 0, stream, args);
    else
      hipLaunchKernelGGL(f32_rows<false>, grid, dim3(kF32T), 0, stream, args);
    return hipGetLastError();
  }
  if (a.vocab < 16384) {
    hipLaunchKernelGGL(generic_rows<uint16_t>, grid, dim3(kGT), 0, stream, args);
    return hipGetLastError();
  }
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 8 == 0);
  // one persistent block per CU (two 64 KB counter buffers)
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu < 1)
    n_cu = 256;
  const int64_t nb = int64_t(n_cu);
  const dim3 pgrid(unsigned(a.n_rows < nb ? a.n_rows : nb));
  if (vec)
    hipLaunchKernelGGL(bf16_hist_rows<true>, pgrid, dim3(kHT), 0, stream, args);
  else
    hipLaunchKernelGGL(bf16_hist_rows<false>, pgrid, dim3(kHT), 0, stream, args);
  return hipGetLastError();
}

}  // namespace rlk
