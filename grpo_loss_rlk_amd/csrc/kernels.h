// Internal launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rlk {

// ----------------------------------------------------------------- logits path
struct RowArgs {
  const void* logits;
  int64_t n_rows, vocab, row_stride;
  const int64_t* targets;
  float temperature, top_p;
  const float* t_row;     // nullable per-row temperature
  const float* p_row;     // nullable per-row top-p
  int32_t top_k;          // top-k for every row (0: off), unless k_row is given
  const int32_t* k_row;   // nullable per-row top-k (0: off; < 0 flags the row)
  const float* kfloor;    // nullable [n_rows]: each row's top-k floor v_k (-inf: none),
                          // set by the launcher when top-k is requested
  float* lp_full;
  float* lp_trunc;
  float* ent_trunc;
  float* ent_full;        // nullable
  int32_t* nsize;         // nullable
  float* thresh;          // nullable
  uint8_t* flags;         // nullable
  float* saved4;          // nullable [n_rows, 4]: log Z_S and E_q over S of z/T, threshold,
                          // 1 when the lp term is live (target in range and kept) else 0
  // fp32 rows produced by the fused LM head (nullable, both or neither):
  // per row, the order key of the max logit and a non-finite flag, written
  // by the producer; read and cleared to 0 here
  uint32_t* zmax_key;
  uint32_t* zbad;
  double* score_stats;    // nullable [n_rows, 2]: the row max m and log Z_S with which
                          // the row's tokens are scored (token_logprob), for live rows
  uint8_t* fallback;      // workspace [n_rows]: rows the histogram path hands on
};

size_t logits_rows_workspace(int64_t n_rows, int64_t vocab, int dtype);
hipError_t launch_logits_rows(const RowArgs& a, int dtype, void* workspace, hipStream_t stream);

// The no-allocation entry point's scratch: one static device array per GPU
// (noalloc.hip), large enough for the logits-in workspace of this many rows.
constexpr int64_t kNoAllocMaxRows = int64_t(1) << 20;
constexpr size_t kNoAllocScratchBytes = 5 * size_t(kNoAllocMaxRows);   // flags + fp32 floors
// This GPU's (the current device's) scratch address, looked up on first use.
hipError_t noalloc_scratch(void** out);

// ------------------------------------------------------------------ GRPO loss
struct GrpoArgs {
  const float* lp_new;
  const float* lp_old;
  const float* lp_ref;        // nullable when kl_coef == 0
  const int64_t* cu;          // device [n_seqs + 1] packed offsets (checked by the kernels)
  int64_t n_seqs, n_tokens;
  const float* rewards;       // one of rewards / advantages
  const float* advantages;
  int32_t group_size;
  float tis_cap, eps_low, eps_high, kl_coef, adv_eps;
  int32_t std_ddof, normalize_std;
  int32_t loss_type, correction, aggregation, filter_zero_adv, baseline;
  float ipo_eps, icepop_lo, icepop_hi;
  float* loss;
  float* grad;
  float* token_loss;          // nullable
  uint8_t* token_flags;       // nullable
  float* metrics;             // nullable
  float* adv_out;             // nullable
  int32_t* status;            // nullable device word: 0 offsets valid, 1 invalid
};

size_t grpo_workspace(int64_t n_tokens, int64_t n_seqs);
hipError_t launch_grpo(const GrpoArgs& a, void* workspace, hipStream_t stream);

}  // namespace rlk
