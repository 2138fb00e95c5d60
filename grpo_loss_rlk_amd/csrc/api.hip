// The C ABI (include/rlk.h): host-side argument validation, workspace sizing
// and dispatch onto the caller's stream. Nothing is launched or written when
// validation fails.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstring>

#include "../../include/rlk.h"
#include "fused_kernels.h"
#include "kernels.h"
#include "sampler_kernels.h"
#include "support_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

rlk_status fail(rlk_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

rlk_status ok() {
  g_last_error[0] = '\0';
  return RLK_OK;
}

rlk_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RLK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

rlk_status check_sampling(float temperature, float top_p, int32_t top_k) {
  if (top_k < 0) return fail(RLK_EINVAL, "top_k=%d must be >= 0 (0: no top-k)", top_k);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(RLK_EINVAL, "temperature=%g must be finite and > 0", double(temperature));
  if (!(top_p > 0.f) || !(top_p <= 1.f))
    return fail(RLK_EINVAL, "top_p=%g must lie in (0, 1]", double(top_p));
  return RLK_OK;
}

rlk_status check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return RLK_OK;
  if (ws == nullptr) return fail(RLK_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(RLK_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(RLK_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return RLK_OK;
}

constexpr int64_t kMaxVocab = int64_t(1) << 24;
// Fused path: the tile GEMM addresses 256 rows of an operand with 32-bit byte
// offsets, so row lengths (strides, padded vocabulary and token counts of the
// transposed backward operands) stay below 2^23 elements.
constexpr int64_t kMaxStride = int64_t(1) << 23;
constexpr int64_t kMaxFusedRows = int64_t(1) << 23;

}  // namespace

extern "C" {

int32_t rlk_abi_version(void) { return 2; }

const char* rlk_status_str(rlk_status s) {
  switch (s) {
    case RLK_OK: return "ok";
    case RLK_EINVAL: return "invalid argument";
    case RLK_EUNSUPPORTED: return "unsupported";
    case RLK_EWORKSPACE: return "workspace too small or misaligned";
    case RLK_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rlk_last_error(void) { return g_last_error; }

// ------------------------------------------------------------------ logits in
size_t rlk_logprob_from_logits_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype) {
  if (n_rows < 0) return 0;
  return rlk::logits_rows_workspace(n_rows, vocab, dtype);
}

}  // extern "C"

namespace {

// Checks of rlk_logprob_from_logits' arguments other than the workspace, and
// the kernel arguments they describe.
rlk_status logits_args(const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab,
                       int64_t row_stride, const int64_t* targets, float temperature,
                       float top_p, const float* temperature_per_row,
                       const float* top_p_per_row, int32_t top_k,
                       const int32_t* top_k_per_row, float* lp_full,
                       float* lp_trunc, float* entropy_trunc, float* entropy_full,
                       int32_t* nucleus_size, float* threshold, uint8_t* flags,
                       rlk::RowArgs* a) {
  if (dtype != RLK_DTYPE_F32 && dtype != RLK_DTYPE_BF16)
    return fail(RLK_EINVAL, "dtype=%d is not RLK_DTYPE_F32 or RLK_DTYPE_BF16", dtype);
  rlk_status s = check_sampling(temperature, top_p, top_k);
  if (s != RLK_OK) return s;
  if (n_rows < 0) return fail(RLK_EINVAL, "n_rows=%lld < 0", (long long)n_rows);
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(RLK_EINVAL, "vocab=%lld outside [1, 2^24]", (long long)vocab);
  if (row_stride < vocab)
    return fail(RLK_EINVAL, "row_stride=%lld < vocab=%lld", (long long)row_stride,
                (long long)vocab);
  if (n_rows == 0) return ok();
  const size_t esz = dtype == RLK_DTYPE_F32 ? 4 : 2;
  if (!logits || !targets || !lp_full || !lp_trunc || !entropy_trunc)
    return fail(RLK_EINVAL, "logits, targets, lp_full, lp_trunc and entropy_trunc are required");
  if (!aligned(logits, esz) || !aligned(targets, 8) || !aligned(lp_full, 4) ||
      !aligned(lp_trunc, 4) || !aligned(entropy_trunc, 4) || !aligned(entropy_full, 4) ||
      !aligned(nucleus_size, 4) || !aligned(threshold, 4) || !aligned(temperature_per_row, 4) ||
      !aligned(top_p_per_row, 4) || !aligned(top_k_per_row, 4))
    return fail(RLK_EINVAL, "an array is not naturally aligned");
  *a = rlk::RowArgs{};
  a->logits = logits;
  a->n_rows = n_rows;
  a->vocab = vocab;
  a->row_stride = row_stride;
  a->targets = targets;
  a->temperature = temperature;
  a->top_p = top_p;
  a->t_row = temperature_per_row;
  a->p_row = top_p_per_row;
  a->top_k = top_k;
  a->k_row = top_k_per_row;
  a->lp_full = lp_full;
  a->lp_trunc = lp_trunc;
  a->ent_trunc = entropy_trunc;
  a->ent_full = entropy_full;
  a->nsize = nucleus_size;
  a->thresh = threshold;
  a->flags = flags;
  return RLK_OK;
}

}  // namespace

extern "C" {

rlk_status rlk_logprob_from_logits(const void* logits, int32_t dtype, int64_t n_rows,
                                   int64_t vocab, int64_t row_stride, const int64_t* targets,
                                   float temperature, float top_p,
                                   const float* temperature_per_row, const float* top_p_per_row,
                                   int32_t top_k, const int32_t* top_k_per_row, float* lp_full,
                                   float* lp_trunc, float* entropy_trunc, float* entropy_full,
                                   int32_t* nucleus_size, float* threshold, uint8_t* flags,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  rlk::RowArgs a;
  rlk_status s = logits_args(logits, dtype, n_rows, vocab, row_stride, targets, temperature,
                             top_p, temperature_per_row, top_p_per_row, top_k, top_k_per_row,
                             lp_full, lp_trunc, entropy_trunc, entropy_full, nucleus_size,
                             threshold, flags, &a);
  if (s != RLK_OK || n_rows == 0) return s;
  s = check_workspace(workspace, workspace_bytes,
                      rlk_logprob_from_logits_workspace_size(n_rows, vocab, dtype));
  if (s != RLK_OK) return s;
  return hip_status(rlk::launch_logits_rows(a, dtype, workspace,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "rlk_logprob_from_logits launch");
}

rlk_status rlk_logprob_from_logits_noalloc(const void* logits, int32_t dtype, int64_t n_rows,
                                           int64_t vocab, int64_t row_stride,
                                           const int64_t* targets, float temperature,
                                           float top_p, const float* temperature_per_row,
                                           const float* top_p_per_row, int32_t top_k,
                                           const int32_t* top_k_per_row, float* lp_full,
                                           float* lp_trunc, float* entropy_trunc,
                                           float* entropy_full, int32_t* nucleus_size,
                                           float* threshold, uint8_t* flags, void* stream) {
  rlk::RowArgs a;
  rlk_status s = logits_args(logits, dtype, n_rows, vocab, row_stride, targets, temperature,
                             top_p, temperature_per_row, top_p_per_row, top_k, top_k_per_row,
                             lp_full, lp_trunc, entropy_trunc, entropy_full, nucleus_size,
                             threshold, flags, &a);
  if (s != RLK_OK) return s;
  if (n_rows > rlk::kNoAllocMaxRows)
    return fail(RLK_EINVAL, "n_rows=%lld exceeds the no-allocation limit of %lld rows",
                (long long)n_rows, (long long)rlk::kNoAllocMaxRows);
  if (n_rows == 0) return s;
  const size_t need = rlk::logits_rows_workspace(n_rows, vocab, dtype);
  if (need > rlk::kNoAllocScratchBytes)
    return fail(RLK_EINVAL, "n_rows=%lld needs %zu bytes of scratch, more than %zu",
                (long long)n_rows, need, rlk::kNoAllocScratchBytes);
  void* scratch = nullptr;
  hipError_t e = rlk::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "rlk_logprob_from_logits_noalloc scratch lookup");
  return hip_status(rlk::launch_logits_rows(a, dtype, scratch,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "rlk_logprob_from_logits_noalloc launch");
}

// ------------------------------------------------------------ retained support
namespace {

// workspace of the nucleus check: lp_full, lp_trunc, entropy_trunc and
// threshold (fp32), nucleus size (int32), flags (uint8), each rounded up to
// 256 bytes, then the logits-in workspace
size_t support_slot(int64_t n, size_t esz) { return (size_t(n) * esz + 255) / 256 * 256; }

}  // namespace

size_t rlk_logprob_from_support_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype,
                                                float check_top_p) {
  if (n_rows < 0 || !(check_top_p > 0.f)) return 0;
  return 5 * support_slot(n_rows, 4) + support_slot(n_rows, 1) +
         rlk::logits_rows_workspace(n_rows, vocab, dtype);
}

rlk_status rlk_logprob_from_support(const void* logits, int32_t dtype, int64_t n_rows,
                                    int64_t vocab, int64_t row_stride, const int64_t* targets,
                                    float temperature, const int64_t* support_offsets,
                                    const int32_t* support_ids, int64_t n_support,
                                    float check_top_p, int32_t check_top_k, float* logprob,
                                    float* entropy, uint8_t* flags, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (dtype != RLK_DTYPE_F32 && dtype != RLK_DTYPE_BF16)
    return fail(RLK_EINVAL, "dtype=%d is not RLK_DTYPE_F32 or RLK_DTYPE_BF16", dtype);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(RLK_EINVAL, "temperature=%g must be finite and > 0", double(temperature));
  const bool check = check_top_p != 0.f;
  if (check && !(check_top_p > 0.f && check_top_p <= 1.f))
    return fail(RLK_EINVAL, "check_top_p=%g must be 0 or lie in (0, 1]", double(check_top_p));
  if (check_top_k < 0 || (check_top_k > 0 && !check))
    return fail(RLK_EINVAL, "check_top_k=%d must be >= 0, and 0 without a check_top_p",
                check_top_k);
  if (n_rows < 0) return fail(RLK_EINVAL, "n_rows=%lld < 0", (long long)n_rows);
  if (n_rows >= (int64_t(1) << 31))
    return fail(RLK_EINVAL, "n_rows=%lld must be below 2^31", (long long)n_rows);
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(RLK_EINVAL, "vocab=%lld outside [1, 2^24]", (long long)vocab);
  if (row_stride < vocab)
    return fail(RLK_EINVAL, "row_stride=%lld < vocab=%lld", (long long)row_stride,
                (long long)vocab);
  if (n_support < 0) return fail(RLK_EINVAL, "n_support=%lld < 0", (long long)n_support);
  if (n_rows == 0) return ok();
  const size_t esz = dtype == RLK_DTYPE_F32 ? 4 : 2;
  if (!logits || !targets || !support_offsets || !logprob || !entropy ||
      (n_support > 0 && !support_ids))
    return fail(RLK_EINVAL,
                "logits, targets, support_offsets, support_ids, logprob and entropy are required");
  if (!aligned(logits, esz) || !aligned(targets, 8) || !aligned(support_offsets, 8) ||
      !aligned(support_ids, 4) || !aligned(logprob, 4) || !aligned(entropy, 4))
    return fail(RLK_EINVAL, "an array is not naturally aligned");
  rlk_status s = check_workspace(
      workspace, workspace_bytes,
      rlk_logprob_from_support_workspace_size(n_rows, vocab, dtype, check_top_p));
  if (s != RLK_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  rlk::SupportArgs a{};
  a.logits = logits;
  a.n_rows = n_rows;
  a.vocab = vocab;
  a.row_stride = row_stride;
  a.targets = targets;
  a.temperature = temperature;
  a.offsets = support_offsets;
  a.ids = support_ids;
  a.n_support = n_support;
  a.lp = logprob;
  a.ent = entropy;
  a.flags = flags;
  if (check) {   // the nucleus of every row, into the workspace
    char* w = static_cast<char*>(workspace);
    const size_t f4 = support_slot(n_rows, 4);
    rlk::RowArgs r{};
    r.logits = logits;
    r.n_rows = n_rows;
    r.vocab = vocab;
    r.row_stride = row_stride;
    r.targets = targets;
    r.temperature = temperature;
    r.top_p = check_top_p;
    r.top_k = check_top_k;
    r.lp_full = reinterpret_cast<float*>(w);
    r.lp_trunc = reinterpret_cast<float*>(w + f4);
    r.ent_trunc = reinterpret_cast<float*>(w + 2 * f4);
    r.thresh = reinterpret_cast<float*>(w + 3 * f4);
    r.nsize = reinterpret_cast<int32_t*>(w + 4 * f4);
    r.flags = reinterpret_cast<uint8_t*>(w + 5 * f4);
    s = hip_status(rlk::launch_logits_rows(r, dtype, w + 5 * f4 + support_slot(n_rows, 1), st),
                   "rlk_logprob_from_support nucleus launch");
    if (s != RLK_OK) return s;
    a.nsize = r.nsize;
    a.thresh = r.thresh;
    a.nflags = r.flags;
  }
  return hip_status(rlk::launch_support_rows(a, dtype, st), "rlk_logprob_from_support launch");
}

// ------------------------------------------------------------------- sampler
size_t rlk_sample_top_p_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype) {
  if (n_rows < 0) return 0;
  // dummy targets (int64), lp_full, lp_trunc, entropy, threshold (fp32), flags,
  // the row max and log Z_S (fp64 pairs), then the logits-in workspace
  return support_slot(n_rows, 8) + 4 * support_slot(n_rows, 4) + support_slot(n_rows, 1) +
         support_slot(n_rows, 16) + rlk::logits_rows_workspace(n_rows, vocab, dtype);
}

rlk_status rlk_sample_top_p(const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab,
                            int64_t row_stride, float temperature, float top_p, int32_t top_k,
                            const float* temperature_per_row, const float* top_p_per_row,
                            const int32_t* top_k_per_row, uint64_t seed, uint32_t offset,
                            const int64_t* row_keys, int64_t* samples, float* logprob,
                            float* entropy, int32_t* nucleus_size, uint8_t* flags,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != RLK_DTYPE_F32 && dtype != RLK_DTYPE_BF16)
    return fail(RLK_EINVAL, "dtype=%d is not RLK_DTYPE_F32 or RLK_DTYPE_BF16", dtype);
  rlk_status s = check_sampling(temperature, top_p, top_k);
  if (s != RLK_OK) return s;
  if (n_rows < 0) return fail(RLK_EINVAL, "n_rows=%lld < 0", (long long)n_rows);
  if (n_rows >= (int64_t(1) << 31))
    return fail(RLK_EINVAL, "n_rows=%lld must be below 2^31", (long long)n_rows);
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(RLK_EINVAL, "vocab=%lld outside [1, 2^24]", (long long)vocab);
  if (row_stride < vocab)
    return fail(RLK_EINVAL, "row_stride=%lld < vocab=%lld", (long long)row_stride,
                (long long)vocab);
  if (n_rows == 0) return ok();
  const size_t esz = dtype == RLK_DTYPE_F32 ? 4 : 2;
  if (!logits || !samples) return fail(RLK_EINVAL, "logits and samples are required");
  if (!aligned(logits, esz) || !aligned(samples, 8) || !aligned(row_keys, 8) ||
      !aligned(logprob, 4) || !aligned(entropy, 4) || !aligned(nucleus_size, 4) ||
      !aligned(temperature_per_row, 4) || !aligned(top_p_per_row, 4) ||
      !aligned(top_k_per_row, 4))
    return fail(RLK_EINVAL, "an array is not naturally aligned");
  s = check_workspace(workspace, workspace_bytes,
                      rlk_sample_top_p_workspace_size(n_rows, vocab, dtype));
  if (s != RLK_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  const size_t f4 = support_slot(n_rows, 4);
  int64_t* zero_t = reinterpret_cast<int64_t*>(w);
  w += support_slot(n_rows, 8);
  float* lp_full = reinterpret_cast<float*>(w);
  float* lp_tr = reinterpret_cast<float*>(w + f4);
  float* ent = reinterpret_cast<float*>(w + 2 * f4);
  float* thr = reinterpret_cast<float*>(w + 3 * f4);
  uint8_t* nfl = reinterpret_cast<uint8_t*>(w + 4 * f4);
  double* stats = reinterpret_cast<double*>(w + 4 * f4 + support_slot(n_rows, 1));
  void* rows_ws = w + 4 * f4 + support_slot(n_rows, 1) + support_slot(n_rows, 16);

  rlk::RowArgs r{};
  r.logits = logits;
  r.n_rows = n_rows;
  r.vocab = vocab;
  r.row_stride = row_stride;
  r.temperature = temperature;
  r.top_p = top_p;
  r.t_row = temperature_per_row;
  r.p_row = top_p_per_row;
  r.top_k = top_k;
  r.k_row = top_k_per_row;
  // 1. each row's nucleus: threshold, entropy, size, flags, and the row max
  // and log Z_S its tokens are scored with (the target is a placeholder)
  s = hip_status(rlk::launch_fill_i64(zero_t, n_rows, 0, st), "rlk_sample_top_p fill");
  if (s != RLK_OK) return s;
  r.targets = zero_t;
  r.lp_full = lp_full;
  r.lp_trunc = lp_tr;
  r.ent_trunc = entropy ? entropy : ent;
  r.nsize = nucleus_size;
  r.thresh = thr;
  r.flags = nfl;
  r.score_stats = stats;
  s = hip_status(rlk::launch_logits_rows(r, dtype, rows_ws, st), "rlk_sample_top_p nucleus");
  if (s != RLK_OK) return s;
  // 2. the draw
  rlk::SampleArgs a{};
  a.logits = logits;
  a.n_rows = n_rows;
  a.vocab = vocab;
  a.row_stride = row_stride;
  a.temperature = temperature;
  a.t_row = temperature_per_row;
  a.seed = seed;
  a.offset = offset;
  a.row_keys = row_keys;
  a.thresh = thr;
  a.nflags = nfl;
  a.score_stats = stats;
  a.samples = samples;
  // 2'. the drawn token scored in the same kernel with the row kernel's own
  // (row max, log Z_S) and token_logprob, so the rollout's logprobs are
  // bitwise those of a training-side call with targets = samples
  a.logprob = logprob;
  a.flags = flags;
  return hip_status(rlk::launch_sample_rows(a, dtype, st), "rlk_sample_top_p draw");
}

// ------------------------------------------------------------------ fused LM head
namespace {

rlk_status check_fused_shapes(const void* hidden, const void* weight, int64_t N, int64_t H,
                              int64_t V, int64_t hs, int64_t ws, const int64_t* targets) {
  if (N < 0) return fail(RLK_EINVAL, "n_rows=%lld < 0", (long long)N);
  if (H < 64 || H % 64 != 0)
    return fail(RLK_EINVAL, "hidden_size=%lld must be a positive multiple of 64", (long long)H);
  if (V < 1 || V > kMaxVocab) return fail(RLK_EINVAL, "vocab=%lld outside [1, 2^24]", (long long)V);
  if (hs < H || ws < H || hs % 8 != 0 || ws % 8 != 0)
    return fail(RLK_EINVAL, "strides (h %lld, w %lld) must be >= hidden_size and multiples of 8",
                (long long)hs, (long long)ws);
  if (hs >= kMaxStride || ws >= kMaxStride)
    return fail(RLK_EINVAL, "strides (h %lld, w %lld) must be below 2^23", (long long)hs,
                (long long)ws);
  if (N >= kMaxFusedRows) return fail(RLK_EINVAL, "n_rows=%lld must be below 2^23", (long long)N);
  if (N == 0) return RLK_OK;
  if (!hidden || !weight || !targets)
    return fail(RLK_EINVAL, "hidden, weight and targets are required");
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(targets, 8))
    return fail(RLK_EINVAL, "hidden and weight must be 16-byte aligned, targets 8-byte aligned");
  return RLK_OK;
}

}  // namespace

size_t rlk_logprob_fused_linear_workspace_size(int64_t n_rows, int64_t hidden_size, int64_t vocab,
                                               float top_p, int32_t top_k) {
  if (n_rows < 0 || vocab < 1) return 0;
  return rlk::fused_fwd_workspace(n_rows, hidden_size, vocab, top_p, top_k);
}

rlk_status rlk_logprob_fused_linear(const void* hidden, const void* weight, int64_t n_rows,
                                    int64_t hidden_size, int64_t vocab, int64_t h_stride,
                                    int64_t w_stride, const int64_t* targets, float temperature,
                                    float top_p, int32_t top_k, float* logprob, float* entropy,
                                    float* saved, int32_t* nucleus_size, uint8_t* flags,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  rlk_status s = check_sampling(temperature, top_p, top_k);
  if (s != RLK_OK) return s;
  s = check_fused_shapes(hidden, weight, n_rows, hidden_size, vocab, h_stride, w_stride, targets);
  if (s != RLK_OK) return s;
  if (n_rows == 0) return ok();
  if (!logprob || !entropy) return fail(RLK_EINVAL, "logprob and entropy are required");
  if (!aligned(logprob, 4) || !aligned(entropy, 4) || !aligned(saved, 4) ||
      !aligned(nucleus_size, 4))
    return fail(RLK_EINVAL, "an output array is not naturally aligned");
  s = check_workspace(
      workspace, workspace_bytes,
      rlk_logprob_fused_linear_workspace_size(n_rows, hidden_size, vocab, top_p, top_k));
  if (s != RLK_OK) return s;
  rlk::FusedFwdArgs a{};
  a.h = reinterpret_cast<const uint16_t*>(hidden);
  a.w = reinterpret_cast<const uint16_t*>(weight);
  a.N = n_rows;
  a.H = hidden_size;
  a.V = vocab;
  a.hs = h_stride;
  a.ws = w_stride;
  a.targets = targets;
  a.c2 = float(1.4426950408889634 / double(temperature));
  a.temperature = temperature;
  a.top_p = top_p;
  a.top_k = top_k;
  a.logprob = logprob;
  a.entropy = entropy;
  a.saved = saved;
  a.nsize = nucleus_size;
  a.flags = flags;
  return hip_status(rlk::launch_fused_fwd(a, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "rlk_logprob_fused_linear launch");
}

size_t rlk_logprob_fused_linear_bwd_workspace_size(int64_t n_rows, int64_t hidden_size,
                                                   int64_t vocab, float top_p) {
  (void)top_p;
  if (n_rows < 0 || hidden_size < 1 || vocab < 1) return 0;
  return rlk::fused_bwd_workspace(n_rows, hidden_size, vocab);
}

rlk_status rlk_logprob_fused_linear_bwd(const void* hidden, const void* weight, int64_t n_rows,
                                        int64_t hidden_size, int64_t vocab, int64_t h_stride,
                                        int64_t w_stride, const int64_t* targets,
                                        const float* saved, const float* grad_logprob,
                                        const float* grad_entropy, float temperature, float top_p,
                                        int32_t top_k, void* grad_hidden, float* grad_weight,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  rlk_status s = check_sampling(temperature, top_p, top_k);
  if (s != RLK_OK) return s;
  s = check_fused_shapes(hidden, weight, n_rows, hidden_size, vocab, h_stride, w_stride, targets);
  if (s != RLK_OK) return s;
  if (vocab >= kMaxFusedRows)
    return fail(RLK_EINVAL, "vocab=%lld must be below 2^23 for the backward", (long long)vocab);
  if (!grad_weight) return fail(RLK_EINVAL, "grad_weight is required");
  if (!aligned(grad_weight, 4)) return fail(RLK_EINVAL, "grad_weight must be 4-byte aligned");
  if (n_rows > 0) {
    if (!saved || !grad_hidden) return fail(RLK_EINVAL, "saved and grad_hidden are required");
    if (!aligned(saved, 4) || !aligned(grad_hidden, 2) || !aligned(grad_logprob, 4) ||
        !aligned(grad_entropy, 4))
      return fail(RLK_EINVAL, "an array is not naturally aligned");
  }
  s = check_workspace(workspace, workspace_bytes,
                      rlk_logprob_fused_linear_bwd_workspace_size(n_rows, hidden_size, vocab,
                                                                  top_p));
  if (s != RLK_OK) return s;
  rlk::FusedBwdArgs a{};
  a.h = reinterpret_cast<const uint16_t*>(hidden);
  a.w = reinterpret_cast<const uint16_t*>(weight);
  a.N = n_rows;
  a.H = hidden_size;
  a.V = vocab;
  a.hs = h_stride;
  a.ws = w_stride;
  a.targets = targets;
  a.saved = saved;
  a.g_lp = grad_logprob;
  a.g_H = grad_entropy;
  a.inv_t = float(1.0 / double(temperature));
  a.dh = reinterpret_cast<uint16_t*>(grad_hidden);
  a.dW = grad_weight;
  return hip_status(rlk::launch_fused_bwd(a, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "rlk_logprob_fused_linear_bwd launch");
}

// ------------------------------------------------------------------ GRPO loss
size_t rlk_grpo_token_loss_workspace_size(int64_t n_tokens, int64_t n_seqs) {
  if (n_tokens < 0 || n_seqs < 0) return 0;
  return rlk::grpo_workspace(n_tokens, n_seqs);
}

rlk_status rlk_grpo_token_loss(const float* lp_new, const float* lp_old, const float* lp_ref,
                               const int64_t* cu_seqlens, int64_t n_seqs, int64_t n_tokens,
                               const float* rewards, const float* advantages, int32_t group_size,
                               const rlk_grpo_params* params, float* loss, float* grad_lp_new,
                               float* token_loss, uint8_t* token_flags, float* metrics,
                               float* adv_out, int32_t* status, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!params) return fail(RLK_EINVAL, "params is NULL");
  // the first layout ends after normalize_std; later fields take their defaults
  constexpr uint32_t kFirstLayout = offsetof(rlk_grpo_params, loss_type);
  if (params->struct_size < kFirstLayout)
    return fail(RLK_EINVAL, "params->struct_size=%u < %u", params->struct_size, kFirstLayout);
  rlk_grpo_params p{};
  p.loss_type = RLK_LOSS_DAPO;
  p.correction = RLK_CORRECTION_TIS;
  p.aggregation = RLK_AGG_TOKEN_MEAN;
  p.filter_zero_adv = 0;
  p.baseline = RLK_BASELINE_MEAN;
  p.ipo_eps = 0.3f;
  p.icepop_lo = 0.5f;
  p.icepop_hi = 2.0f;
  std::memcpy(&p, params, params->struct_size < sizeof(p) ? params->struct_size : sizeof(p));
  if (p.loss_type < RLK_LOSS_DAPO || p.loss_type > RLK_LOSS_TIS_PG)
    return fail(RLK_EINVAL, "loss_type=%d is not an RLK_LOSS_* value", p.loss_type);
  if (p.correction != RLK_CORRECTION_TIS && p.correction != RLK_CORRECTION_MIS)
    return fail(RLK_EINVAL, "correction=%d is not an RLK_CORRECTION_* value", p.correction);
  if (p.aggregation != RLK_AGG_TOKEN_MEAN && p.aggregation != RLK_AGG_PROMPT_MEAN)
    return fail(RLK_EINVAL, "aggregation=%d is not an RLK_AGG_* value", p.aggregation);
  if (p.filter_zero_adv != 0 && p.filter_zero_adv != 1)
    return fail(RLK_EINVAL, "filter_zero_adv must be 0 or 1");
  if (p.baseline != RLK_BASELINE_MEAN && p.baseline != RLK_BASELINE_LENGTH)
    return fail(RLK_EINVAL, "baseline=%d is not an RLK_BASELINE_* value", p.baseline);
  if (!(p.ipo_eps > 0.f) || !std::isfinite(p.ipo_eps))
    return fail(RLK_EINVAL, "ipo_eps must be finite and > 0");
  if (!(p.icepop_lo > 0.f) || !(p.icepop_hi >= p.icepop_lo) || !std::isfinite(p.icepop_hi))
    return fail(RLK_EINVAL, "the IcePop band must satisfy 0 < icepop_lo <= icepop_hi < inf");
  if (!(p.tis_cap > 0.f) || !std::isfinite(p.tis_cap))
    return fail(RLK_EINVAL, "tis_cap must be finite and > 0");
  if (!(p.eps_low >= 0.f && p.eps_low < 1.f)) return fail(RLK_EINVAL, "eps_low must lie in [0, 1)");
  if (!(p.eps_high >= 0.f) || !std::isfinite(p.eps_high))
    return fail(RLK_EINVAL, "eps_high must be finite and >= 0");
  if (!(p.kl_coef >= 0.f) || !std::isfinite(p.kl_coef))
    return fail(RLK_EINVAL, "kl_coef must be finite and >= 0");
  if (!(p.adv_eps >= 0.f) || !std::isfinite(p.adv_eps))
    return fail(RLK_EINVAL, "adv_eps must be finite and >= 0");
  if (p.std_ddof != 0 && p.std_ddof != 1) return fail(RLK_EINVAL, "std_ddof must be 0 or 1");
  if (n_seqs < 1) return fail(RLK_EINVAL, "n_seqs=%lld < 1", (long long)n_seqs);
  if (n_seqs > (int64_t(1) << 31)) return fail(RLK_EINVAL, "n_seqs=%lld too large", (long long)n_seqs);
  if (!cu_seqlens) return fail(RLK_EINVAL, "cu_seqlens is NULL");
  if (!aligned(cu_seqlens, 8)) return fail(RLK_EINVAL, "cu_seqlens is not 8-byte aligned");
  if (n_tokens < 0 || n_tokens > (int64_t(1) << 40))
    return fail(RLK_EINVAL, "n_tokens=%lld outside [0, 2^40]", (long long)n_tokens);
  if (!aligned(status, 4)) return fail(RLK_EINVAL, "status is not 4-byte aligned");
  if ((rewards == nullptr) == (advantages == nullptr))
    return fail(RLK_EINVAL, "exactly one of rewards / advantages must be given");
  if (rewards || p.aggregation == RLK_AGG_PROMPT_MEAN) {
    if (group_size < 1 || n_seqs % group_size != 0)
      return fail(RLK_EINVAL, "group_size=%d must be >= 1 and divide n_seqs=%lld", group_size,
                  (long long)n_seqs);
  }
  if (rewards) {
    if (p.normalize_std && group_size - p.std_ddof < 1)
      return fail(RLK_EINVAL, "group_size=%d too small for a std with ddof=%d", group_size,
                  p.std_ddof);
  }
  if (!loss) return fail(RLK_EINVAL, "loss is required");
  if (n_tokens > 0 && (!lp_new || !lp_old || !grad_lp_new))
    return fail(RLK_EINVAL, "lp_new, lp_old and grad_lp_new are required");
  if (n_tokens > 0 && p.kl_coef != 0.f && !lp_ref)
    return fail(RLK_EINVAL, "lp_ref is required when kl_coef != 0");
  if (!aligned(lp_new, 4) || !aligned(lp_old, 4) || !aligned(lp_ref, 4) || !aligned(loss, 4) ||
      !aligned(grad_lp_new, 4) || !aligned(token_loss, 4) || !aligned(metrics, 4) ||
      !aligned(adv_out, 4) || !aligned(rewards, 4) || !aligned(advantages, 4))
    return fail(RLK_EINVAL, "an array is not naturally aligned");
  rlk_status s = check_workspace(workspace, workspace_bytes,
                                 rlk_grpo_token_loss_workspace_size(n_tokens, n_seqs));
  if (s != RLK_OK) return s;

  rlk::GrpoArgs a{};
  a.lp_new = lp_new;
  a.lp_old = lp_old;
  a.lp_ref = p.kl_coef != 0.f ? lp_ref : nullptr;
  a.cu = cu_seqlens;
  a.n_seqs = n_seqs;
  a.n_tokens = n_tokens;
  a.rewards = rewards;
  a.advantages = advantages;
  a.group_size = group_size;
  a.tis_cap = p.tis_cap;
  a.eps_low = p.eps_low;
  a.eps_high = p.eps_high;
  a.kl_coef = p.kl_coef;
  a.adv_eps = p.adv_eps;
  a.std_ddof = p.std_ddof;
  a.normalize_std = p.normalize_std;
  a.loss_type = p.loss_type;
  a.correction = p.correction;
  a.aggregation = p.aggregation;
  a.filter_zero_adv = p.filter_zero_adv;
  a.baseline = p.baseline;
  a.ipo_eps = p.ipo_eps;
  a.icepop_lo = p.icepop_lo;
  a.icepop_hi = p.icepop_hi;
  a.loss = loss;
  a.grad = grad_lp_new;
  a.token_loss = token_loss;
  a.token_flags = token_flags;
  a.metrics = metrics;
  a.adv_out = adv_out;
  a.status = status;
  return hip_status(rlk::launch_grpo(a, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "rlk_grpo_token_loss launch");
}

}  // extern "C"
