// Logits in: full and top-p truncated log-probability and entropy per row.
//
// What is computed (Qwen3-8B VIME train-rollout consistency page, "ROCm MI300X
// and gfx942": temperature > 0, top-p in (0, 1], the complete nucleus is
// scored, top-p = 1 is the full vocabulary, a monitoring entropy is fused
// with the logprob): for a row z, d_i = (z_i - max z)/T, the full softmax
// statistics, the nucleus S = {z >= tau} with tau the lowest row value whose
// strictly-higher mass is below p (all ties kept), and the statistics of the
// distribution renormalised over S.
//
// Two kernels, chosen per call by dtype and vocabulary size only (never by the
// number of rows, so a row's result does not depend on its batch):
//
//  * bf16_hist_rows: bf16 rows with V >= 16384. A bf16 value has only 65536
//    bit patterns, so one streaming pass that counts each pattern in LDS
//    (16-bit counters, two per 32-bit word, 128 KB) captures the whole row.
//    Everything after that -- max, Z, entropy, the top-p cut, the truncated
//    sums -- is exact arithmetic over the distinct values (fp64, fixed
//    order), so HBM is read once at 5 VALU ops per element. A 16-bit counter
//    that would exceed 65535 (one value holding > 43% of a long row) is
//    detected by a checksum and the row is handed to the generic kernel.
//
//  * generic_rows: any dtype and size. Multi-pass over the row: max, then
//    exp / Z / entropy with a 12-bit radix histogram of fixed-point masses,
//    then two refinement rounds (10 + 10 bits) restricted to the boundary
//    bin, then the truncated sums. Masses are integers (2^-39 of the max
//    element's mass) so LDS atomics are order-free and the cut is bitwise
//    deterministic.
#include "common.h"
#include "kernels.h"

namespace rlk {

namespace {

constexpr uint8_t kOutside = 1, kBadTarget = 2, kNonFinite = 4, kBoundary = 8, kBadParam = 16;
constexpr double kBoundaryEps = 1e-6;

RLK_DEV bool param_ok(float T, float p) {
  return T > 0.f && T <= 3.4e38f && p > 0.f && p <= 1.f;  // NaN fails every compare
}

RLK_DEV void store_row(const RowArgs& a, int64_t row, float lp_full, float lp_trunc,
                       float h_full, float h_trunc, int32_t size, float tau, uint8_t flags) {
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
  store_row(a, row, nan, nan, nan, nan, 0, nan, flags);
}

// ===========================================================================
// bf16 pattern-count histogram kernel
// ===========================================================================
constexpr int kHT = 1024;              // threads per row
constexpr int kHWords = 32768;         // word w: lo16 = count(code w), hi16 = count(code 0x8000|w)
constexpr int kWordsPerThread = kHWords / kHT;
constexpr uint32_t kInfW = 0x7f80;     // codes with w >= 0x7f80 are inf / NaN

RLK_DEV void hist_add(uint32_t* hist, uint32_t code) {
  atomicAdd(&hist[code & 0x7fffu], (code & 0x8000u) ? 0x10000u : 1u);
}

// Both bf16 patterns of a 32-bit word: word index = magnitude bits, the sign
// picks the 16-bit half (increment 1 or 65536 = sign * 65535 + 1).
RLK_DEV void hist_add2(uint32_t* hist, uint32_t x) {
  char* base = reinterpret_cast<char*>(hist);
  atomicAdd(reinterpret_cast<uint32_t*>(base + ((x << 2) & 0x1fffcu)),
            __builtin_amdgcn_ubfe(x, 15, 1) * 65535u + 1u);
  atomicAdd(reinterpret_cast<uint32_t*>(base + ((x >> 14) & 0x1fffcu)), (x >> 31) * 65535u + 1u);
}

// Merged key order over bf16 patterns: key = code | 0x8000 for positive codes,
// ~code & 0xffff for negative ones; -0 (key 0x7fff) is folded into +0 (0x8000).
// Returns the count of the value with this key, and the value.
RLK_DEV uint32_t key_count(const uint32_t* hist, uint32_t key, float* value) {
  if (key >= 0x8000u) {
    const uint32_t c = key - 0x8000u;
    uint32_t n = hist[c] & 0xffffu;
    if (c == 0) n += hist[0] >> 16;   // -0 joins +0
    *value = bf16_to_f32(uint16_t(c));
    return n;
  }
  const uint32_t c = (~key) & 0xffffu;   // negative code
  *value = bf16_to_f32(uint16_t(c));
  if (c == 0x8000u) return 0;            // -0 already counted with +0
  return hist[c & 0x7fffu] >> 16;
}

RLK_DEV uint32_t bf16_key_merged(uint16_t code) {
  if (code == 0x8000u) code = 0;
  return (code & 0x8000u) ? ((~uint32_t(code)) & 0xffffu) : (uint32_t(code) | 0x8000u);
}

constexpr int kHW = kHT / kWave;       // waves per block
constexpr int kPF = 4;                  // 16-byte vectors per thread prefetched for the next row

// exp((v - m) / T) for a bf16 value v and the row max m, in fp32. dv = v - m
// is exact (two bf16 values). With c = log2(e)/T split as c_hi + c_lo, the
// exponent x = dv*c is rounded to x_hi = fl(dv*c_hi) and its residual
// r = (dv*c_hi - x_hi) + dv*c_lo is recovered exactly enough by an fma, so
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

RLK_DEV float code_mass(float dv, MassScale k) {
  const float xh = dv * k.c_hi;
  const float r = fmaf(dv, k.c_hi, -xh) + dv * k.c_lo;
  const float e = exp2f(xh);
  return fmaf(e, r * 0.69314718f, e);
}

RLK_DEV void hist_add8(uint32_t* hist, const uint4& q) {
  hist_add2(hist, q.x);
  hist_add2(hist, q.y);
  hist_add2(hist, q.z);
  hist_add2(hist, q.w);
}

// Per-row scalars handed from the block's reductions to the single thread
// that forms the outputs.
struct RowFinish {
  double Z, S, Zs, Ss, Mgt, invT;
  float m, p;
  uint32_t tau_key;
  int size;
  bool cut, pending;
  uint8_t flags;
  uint16_t cy;
  int64_t row;
};

RLK_DEV float merged_key_value(uint32_t key) {
  if (key == 0x8000u) return 0.f;
  return key > 0x8000u ? bf16_to_f32(uint16_t(key - 0x8000u)) : bf16_to_f32(uint16_t(~key & 0xffffu));
}

RLK_DEV void finish_row(const RowArgs& a, const RowFinish& f) {
  uint8_t flags = f.flags;
  const double logZ = log(f.Z), logZs = log(f.Zs);
  const float h_full = float(logZ - f.S / f.Z);
  const float h_trunc = float(logZs - f.Ss / f.Zs);
  float lpf = __builtin_nanf(""), lpt = __builtin_nanf("");
  if (!(flags & kBadTarget)) {
    const float vy = bf16_to_f32(f.cy);
    if (vy == -INFINITY) {
      lpf = -INFINITY;
      lpt = -INFINITY;
      flags |= kOutside;
    } else {
      const double dy = double(vy - f.m) * f.invT;
      lpf = float(dy - logZ);
      if (!f.cut || bf16_key_merged(f.cy) >= f.tau_key) {
        lpt = float(dy - logZs);
      } else {
        lpt = -INFINITY;
        flags |= kOutside;
      }
    }
  }
  float tau = -INFINITY;
  if (f.cut) {
    tau = merged_key_value(f.tau_key);
    const double pp = double(f.p);
    if (fabs(f.Mgt / f.Z - pp) <= kBoundaryEps || fabs(f.Zs / f.Z - pp) <= kBoundaryEps)
      flags |= kBoundary;
  }
  store_row(a, f.row, lpf, lpt, h_full, h_trunc, f.size, tau, flags);
}

// One persistent block per CU walks rows blockIdx.x, +gridDim.x, ... While a
// row's histogram is post-processed, the first kPF*kHT vectors of the next row
// are already in flight, so HBM keeps streaming. Every reduction is a DPP wave
// scan plus one barrier and a fixed-order fold over the 16 wave partials.
template <bool kVec>
__global__ __launch_bounds__(kHT) void bf16_hist_rows(RowArgs a) {
  __shared__ uint32_t hist[kHWords];
  __shared__ int s_i[2][8][kHW];
  __shared__ double s_d[2][4][kHW];
  __shared__ double b_d[4];
  __shared__ int b_i[2];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t V = a.vocab;
  const int64_t nvec = kVec ? (V >> 3) : 0;

  {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (int i = tid; i < kHWords / 4; i += kHT) h4[i] = make_uint4(0, 0, 0, 0);
  }
  uint4 pf[kPF];
  int64_t row = blockIdx.x;
  if (kVec && row < a.n_rows) {
    const uint4* v4 = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(a.logits) + row * a.row_stride);
#pragma unroll
    for (int u = 0; u < kPF; ++u)
      if (tid + u * kHT < nvec) pf[u] = v4[tid + u * kHT];
  }
  __shared__ RowFinish fin;     // written and read by thread 0 only
  if (tid == 0) fin.pending = false;
  __syncthreads();

  for (; row < a.n_rows; row += gridDim.x) {
    const uint16_t* rowp = reinterpret_cast<const uint16_t*>(a.logits) + row * a.row_stride;
    const int64_t y = a.targets[row];
    const bool y_ok = y >= 0 && y < V;
    uint16_t cy = 0;
    if (tid == 0 && y_ok) cy = rowp[y];

    // ---- one streaming pass: count every bf16 pattern of the row ----
    if (kVec) {
      const uint4* v4 = reinterpret_cast<const uint4*>(rowp);
#pragma unroll
      for (int u = 0; u < kPF; ++u)
        if (tid + u * kHT < nvec) hist_add8(hist, pf[u]);
      int64_t i = tid + kPF * kHT;
      for (; i + 3 * kHT < nvec; i += 4 * kHT) {
        uint4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = v4[i + u * kHT];
#pragma unroll
        for (int u = 0; u < 4; ++u) hist_add8(hist, q[u]);
      }
      for (; i < nvec; i += kHT) hist_add8(hist, v4[i]);
      for (int64_t j = (nvec << 3) + tid; j < V; j += kHT) hist_add(hist, rowp[j]);
    } else {
      for (int64_t j = tid; j < V; j += kHT) hist_add(hist, rowp[j]);
    }
    __syncthreads();

    // ---- the next row's first vectors go in flight now ----
    const int64_t nxt = row + gridDim.x;
    if (kVec && nxt < a.n_rows) {
      const uint4* v4n = reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint16_t*>(a.logits) + nxt * a.row_stride);
#pragma unroll
      for (int u = 0; u < kPF; ++u)
        if (tid + u * kHT < nvec) pf[u] = v4n[tid + u * kHT];
    }

    // ---- phase A: checksum, occupied word range, non-finite detection ----
    // thread t owns words t + kHT*j; a bit mask of its nonzero finite words
    // gives the range [wmin, wmax] every later phase is limited to.
    {
      uint32_t tot = 0, nzmask = 0;
      int nonfin = 0, nneg = 0;
#pragma unroll
      for (int j = 0; j < kWordsPerThread - 1; ++j) {
        const uint32_t x = hist[tid + j * kHT];
        tot = __builtin_amdgcn_sad_u16(x, 0u, tot);
        nzmask |= x ? (1u << j) : 0u;
      }
      {
        const int w = tid + (kWordsPerThread - 1) * kHT;
        const uint32_t x = hist[w];
        tot = __builtin_amdgcn_sad_u16(x, 0u, tot);
        if (w < int(kInfW)) {
          nzmask |= x ? (1u << (kWordsPerThread - 1)) : 0u;
        } else {
          if (x & 0xffffu) nonfin = 1;                  // +inf or NaN
          if ((x >> 16) && w > int(kInfW)) nonfin = 1;  // NaN
          if (w == int(kInfW)) nneg = int(x >> 16);     // -inf
        }
      }
      const int wmax = nzmask ? tid + kHT * (31 - __clz(nzmask)) : -1;
      const int wmin = nzmask ? tid + kHT * (__ffs(nzmask) - 1) : 0x7fff;
      const int t_w = wave_total(int(tot));
      const int nneg_w = wave_total(nneg);
      const int wmax_w = wave_max_i32(wmax);
      const int wmin_w = wave_min_i32(wmin);
      const int nonfin_w = wave_max_i32(nonfin);
      if (lane == 0) {
        s_i[0][0][wid] = t_w;
        s_i[0][1][wid] = nneg_w;
        s_i[0][2][wid] = wmax_w;
        s_i[0][3][wid] = wmin_w;
        s_i[0][4][wid] = nonfin_w;
      }
    }
    __syncthreads();
    const int tot = fold_partials(s_i[0][0], kHW);
    const int nneg = fold_partials(s_i[0][1], kHW);
    const int wmax = wave_max_i32(lane < kHW ? s_i[0][2][lane] : -1);
    const int wmin = wave_min_i32(lane < kHW ? s_i[0][3][lane] : 0x7fff);
    const int nonfin = wave_max_i32(lane < kHW ? s_i[0][4][lane] : 0);

    const float T = a.t_row ? a.t_row[row] : a.temperature;
    const float p = a.p_row ? a.p_row[row] : a.top_p;
    uint8_t flags = 0;
    if (!y_ok) flags |= kBadTarget;
    if (!param_ok(T, p)) flags |= kBadParam;
    if (nonfin || wmax < 0) flags |= kNonFinite;
    const bool overflow = tot != int(V);    // a 16-bit counter wrapped: the generic kernel redoes it
    const bool live = !overflow && !(flags & (kNonFinite | kBadParam));
    if (tid == 0) {
      a.fallback[row] = overflow ? 1 : 0;
      if (!overflow && !live) store_nan_row(a, row, flags);
    }

    if (live) {
      // largest positive pattern (highest word with a nonzero low half),
      // searched down from wmax; if there is none, the smallest-magnitude
      // negative one, searched up from wmin
      int maxpos = -1, minneg = 0x8000;
      for (int k = 0; k <= wmax - wmin && maxpos < 0; k += kHT) {
        const int w = wmax - k - tid;
        const uint32_t x = hist[w >= wmin ? w : wmin];
        const int c = (w >= wmin && (x & 0xffffu)) ? w : -1;
        const int cw = wave_max_i32(c);
        if (lane == 0) s_i[1][2][wid] = cw;
        __syncthreads();
        maxpos = wave_max_i32(lane < kHW ? s_i[1][2][lane] : -1);
        __syncthreads();
      }
      for (int k = 0; k <= wmax - wmin && maxpos < 0 && minneg == 0x8000; k += kHT) {
        const int w = wmin + k + tid;
        const uint32_t x = hist[w <= wmax ? w : wmax];
        const int c = (w <= wmax && (x >> 16)) ? w : 0x8000;
        const int cw = wave_min_i32(c);
        if (lane == 0) s_i[1][3][wid] = cw;
        __syncthreads();
        minneg = wave_min_i32(lane < kHW ? s_i[1][3][lane] : 0x8000);
        __syncthreads();
      }
      float mval;
      uint32_t kmax;
      if (maxpos >= 0) {
        mval = bf16_to_f32(uint16_t(maxpos));
        kmax = 0x8000u + uint32_t(maxpos);
      } else if (minneg == 0) {      // only -0 at the top: same value as +0
        mval = 0.f;
        kmax = 0x8000u;
      } else {
        mval = bf16_to_f32(uint16_t(0x8000 | minneg));
        kmax = 0x7fffu - uint32_t(minneg);
      }
      const double invT = 1.0 / double(T);
      const float invTf = float(invT);
      const MassScale ks = mass_scale(invT);

      // ---- phase B: Z and sum e*d over the distinct finite values ----
      {
        double zt = 0.0, st = 0.0;
        for (int w = wmin + tid; w <= wmax; w += kHT) {
          const uint32_t x = hist[w];
          if (x & 0xffffu) {
            const float dv = bf16_to_f32(uint16_t(w)) - mval;
            const float e = code_mass(dv, ks) * float(x & 0xffffu);
            zt += double(e);
            st += double(e) * double(dv * invTf);
          }
          if (x >> 16) {
            const float dv = bf16_to_f32(uint16_t(0x8000 | w)) - mval;
            const float e = code_mass(dv, ks) * float(x >> 16);
            zt += double(e);
            st += double(e) * double(dv * invTf);
          }
        }
        zt = wave_total(zt);
        st = wave_total(st);
        if (lane == 0) {
          s_d[0][0][wid] = zt;
          s_d[0][1][wid] = st;
        }
      }
      __syncthreads();
      const double Z = fold_partials(s_d[0][0], kHW);
      const double S = fold_partials(s_d[0][1], kHW);

      // ---- phase C: top-p cut, walking merged keys down from the max ----
      double Zs = Z, Ss = S, Mgt = 0.0;
      uint32_t tau_key = 0;
      int size = int(V) - nneg;
      const bool cut = p < 1.f;
      if (cut) {
        const double thr = double(p) * Z;
        double cz = 0.0, cs = 0.0;
        int cn = 0;
        bool found = false;
        int par = 0;
        for (int k0 = int(kmax); !found && k0 >= 0x0080; k0 -= kHT, par ^= 1) {
          const int key = k0 - tid;
          double mass = 0.0, ms = 0.0;
          int n = 0;
          if (key >= 0x0080) {              // keys below 0x0080 are -inf / NaN
            float v;
            n = int(key_count(hist, uint32_t(key), &v));
            if (n) {
              const float dv = v - mval;
              const float e = code_mass(dv, ks) * float(n);
              mass = double(e);
              ms = mass * double(dv * invTf);
            }
          }
          const double iz = wave_scan_incl(mass), is = wave_scan_incl(ms);
          const int in = wave_scan_incl(n);
          if (lane == kWave - 1) {
            s_d[1][2 * par][wid] = iz;
            s_d[1][2 * par + 1][wid] = is;
            s_i[1][par][wid] = in;
          }
          __syncthreads();
          // wave partials in lanes 0..kHW-1: exclusive prefixes and the
          // inclusive value exactly as the crossing wave's last lane forms it
          const double pz = lane < kHW ? s_d[1][2 * par][lane] : 0.0;
          const double ps = lane < kHW ? s_d[1][2 * par + 1][lane] : 0.0;
          const int pn = lane < kHW ? s_i[1][par][lane] : 0;
          const double ez = wave_shift_up(wave_scan_incl(pz));
          const double es = wave_shift_up(wave_scan_incl(ps));
          const int en = wave_shift_up(wave_scan_incl(pn));
          const uint64_t wcross = __ballot(lane < kHW && cz + (ez + pz) >= thr);
          const int cross_wave = wcross ? __ffsll((unsigned long long)wcross) - 1 : -1;
          const double bz = readlane_f64(ez, kHW - 1) + readlane_f64(pz, kHW - 1);
          const double bs = readlane_f64(es, kHW - 1) + readlane_f64(ps, kHW - 1);
          const int bn = int(readlane_u32(uint32_t(en), kHW - 1)) + int(readlane_u32(uint32_t(pn), kHW - 1));
          if (cross_wave >= 0) {
            if (wid == cross_wave) {
              const double wbz = readlane_f64(ez, cross_wave);
              const double wbs = readlane_f64(es, cross_wave);
              const int wbn = int(readlane_u32(uint32_t(en), cross_wave));
              const double incl = cz + (wbz + iz);
              const uint64_t bal = __ballot(incl >= thr);
              const int first = __ffsll((unsigned long long)bal) - 1;
              if (lane == first) {
                b_d[0] = incl;
                b_d[1] = cs + (wbs + is);
                b_d[2] = incl - mass;
                b_i[0] = key;
                b_i[1] = cn + wbn + in;
              }
            }
            __syncthreads();
            Zs = b_d[0];
            Ss = b_d[1];
            Mgt = b_d[2];
            tau_key = uint32_t(b_i[0]);
            size = b_i[1];
            found = true;
          } else {
            cz += bz;
            cs += bs;
            cn += bn;
          }
        }
        if (!found) {   // rounding left the mass just short of p: keep every finite value
          Zs = cz;
          Ss = cs;
          Mgt = cz;
          tau_key = 0x0080;
          size = cn;
        }
      }

      // the row's scalars, finished below once the counters are released
      if (tid == 0) {
        fin.Z = Z; fin.S = S; fin.Zs = Zs; fin.Ss = Ss; fin.Mgt = Mgt;
        fin.m = mval; fin.invT = invT; fin.p = p; fin.tau_key = tau_key;
        fin.size = size; fin.cut = cut; fin.flags = flags; fin.cy = cy; fin.row = row;
        fin.pending = true;
      }
    }

    // ---- clear the counters for the next row: every nonzero word lies in
    // [wmin, wmax] or among the inf/NaN words ----
    __syncthreads();
    for (int w = wmin + tid; w <= wmax; w += kHT) hist[w] = 0;
    if (tid + (kWordsPerThread - 1) * kHT >= int(kInfW)) hist[tid + (kWordsPerThread - 1) * kHT] = 0;
    __syncthreads();
    // thread 0 finishes the row (fp64 logs) while the other waves start streaming
    if (tid == 0 && fin.pending) {
      finish_row(a, fin);
      fin.pending = false;
    }
  }
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
RLK_DEV int walk_down(const uint64_t* bins, int start, uint64_t thr, uint64_t carry,
                      uint64_t* above, uint64_t* su64, int* si, uint64_t* bslot) {
  for (int base = start; base >= 0; base -= kGT) {
    const int b = base - int(threadIdx.x);
    const uint64_t v = b >= 0 ? bins[b] : 0ull;
    uint64_t tot;
    const uint64_t incl = block_inclusive_scan(v, su64, &tot);
    const int cand = (v != 0ull && carry + incl >= thr) ? int(threadIdx.x) : kGT;
    const int first = block_min(cand, si);
    if (first < kGT) {
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

template <typename T>
__global__ __launch_bounds__(kGT) void generic_rows(RowArgs a, int only_fallback) {
  __shared__ uint64_t hist[kBins1];
  __shared__ double sd[kGT / kWave];
  __shared__ uint64_t su64[kGT / kWave];
  __shared__ int si[kGT / kWave];
  __shared__ float sf[kGT / kWave];
  __shared__ uint64_t bslot;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (only_fallback && a.fallback[row] == 0) return;
  const int64_t V = a.vocab;
  const T* rowp = reinterpret_cast<const T*>(a.logits) + row * a.row_stride;

  float Tv = a.t_row ? a.t_row[row] : a.temperature;
  float p = a.p_row ? a.p_row[row] : a.top_p;
  const int64_t y = a.targets[row];
  uint8_t flags = 0;
  if (y < 0 || y >= V) flags |= kBadTarget;
  if (!param_ok(Tv, p)) {
    if (tid == 0) store_nan_row(a, row, flags | kBadParam);
    return;
  }

  // ---- pass 1: max, finite count, non-finite detection ----
  float mx = -INFINITY;
  int bad = 0;
  uint32_t nfin = 0;
  for (int64_t i = tid; i < V; i += kGT) {
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
  const bool cut = p < 1.f;

  // ---- pass 2: Z, sum e*d, round-1 histogram of fixed-point masses ----
  for (int i = tid; i < kBins1; i += kGT) hist[i] = 0ull;
  __syncthreads();
  double zt = 0.0, st = 0.0;
  uint64_t wt = 0;
  for (int64_t i = tid; i < V; i += kGT) {
    const float z = load_val(rowp, i);
    if (!(z > -INFINITY)) continue;
    double d;
    const float e = mass_of(z, m, invT, &d);
    zt += double(e);
    st += double(e) * d;
    if (cut) {
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
    const uint64_t W = block_sum(wt, su64);
    const uint64_t thr = uint64_t(ceil(double(p) * double(W)));
    // round 1
    uint64_t above = 0;
    int d1 = walk_down(hist, kBins1 - 1, thr, 0ull, &above, su64, si, &bslot);
    if (d1 < 0) d1 = 0;   // unreachable: the total mass reaches thr
    // round 2
    __syncthreads();
    for (int i = tid; i < kBins2; i += kGT) hist[i] = 0ull;
    __syncthreads();
    for (int64_t i = tid; i < V; i += kGT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = f32_key(z);
      if (int(k >> 20) != d1) continue;
      double d;
      const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
      if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(k >> 10) & 0x3ffu]),
                       (unsigned long long)w);
    }
    __syncthreads();
    int d2 = walk_down(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
    if (d2 < 0) d2 = 0;
    // round 3
    __syncthreads();
    for (int i = tid; i < kBins2; i += kGT) hist[i] = 0ull;
    __syncthreads();
    const uint32_t pre = (uint32_t(d1) << 10) | uint32_t(d2);
    for (int64_t i = tid; i < V; i += kGT) {
      const float z = load_val(rowp, i);
      if (!(z > -INFINITY)) continue;
      const uint32_t k = f32_key(z);
      if ((k >> 10) != pre) continue;
      double d;
      const uint64_t w = fixed_mass(mass_of(z, m, invT, &d));
      if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[k & 0x3ffu]),
                       (unsigned long long)w);
    }
    __syncthreads();
    int d3 = walk_down(hist, kBins2 - 1, thr, above, &above, su64, si, &bslot);
    if (d3 < 0) d3 = 0;
    tau_key = (pre << 10) | uint32_t(d3);
    const uint64_t at = hist[d3];
    if (tid == 0) {
      const double pp = double(p);
      if (fabs(double(above) / double(W) - pp) <= kBoundaryEps ||
          fabs(double(above + at) / double(W) - pp) <= kBoundaryEps)
        flags |= kBoundary;
    }
    // final pass: truncated sums over S = {key >= tau}
    double zs = 0.0, ss = 0.0;
    uint32_t cnt = 0;
    for (int64_t i = tid; i < V; i += kGT) {
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
        const double dy = (double(zy) - m) * invT;
        lpf = float(dy - logZ);
        if (!cut || f32_key(zy) >= tau_key) {
          lpt = float(dy - logZs);
        } else {
          lpt = -INFINITY;
          flags |= kOutside;
        }
      }
    }
    const float tau = cut ? key_f32(tau_key) : -INFINITY;
    store_row(a, row, lpf, lpt, float(logZ - S / Z), float(logZs - Ss / Zs), int32_t(size), tau,
              flags);
  }
}

}  // namespace

size_t logits_rows_workspace(int64_t n_rows, int64_t vocab, int dtype) {
  (void)vocab;
  (void)dtype;
  return size_t((n_rows + 255) / 256 * 256);
}

hipError_t launch_logits_rows(const RowArgs& a, int dtype, void* workspace, hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  RowArgs args = a;
  args.fallback = reinterpret_cast<uint8_t*>(workspace);
  const dim3 grid(unsigned(a.n_rows));
  if (dtype == 0) {  // fp32
    hipLaunchKernelGGL(generic_rows<float>, grid, dim3(kGT), 0, stream, args, 0);
    return hipGetLastError();
  }
  if (a.vocab < 16384) {
    hipLaunchKernelGGL(generic_rows<uint16_t>, grid, dim3(kGT), 0, stream, args, 0);
    return hipGetLastError();
  }
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 8 == 0);
  // one persistent block per CU (the 128 KB histogram allows one per CU anyway)
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu < 1)
    n_cu = 256;
  const dim3 pgrid(unsigned(a.n_rows < n_cu ? a.n_rows : n_cu));
  if (vec)
    hipLaunchKernelGGL(bf16_hist_rows<true>, pgrid, dim3(kHT), 0, stream, args);
  else
    hipLaunchKernelGGL(bf16_hist_rows<false>, pgrid, dim3(kHT), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.vocab > 65535) {   // a 16-bit counter can only overflow in rows this long
    hipLaunchKernelGGL(generic_rows<uint16_t>, grid, dim3(kGT), 0, stream, args, 1);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace rlk
