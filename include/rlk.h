/*
 * rlk -- token log-probabilities, entropy and the GRPO token loss on MI355X (gfx950).
 *
 * A small C ABI over hand-written HIP kernels. It computes, per sampled
 * response token, the log-probability and entropy of the policy's vocabulary
 * softmax, in the temperature-scaled, top-p-truncated and renormalised form
 * that rollout and training must agree on bitwise (RL-Kernel ROCm sparse
 * performance page, profile paragraph: a consistency run fails on any
 * compared logprob that is not bitwise equal), the fused LM-head form with its
 * backward, and the GRPO/DAPO token loss built on them.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.    Arrays are DEVICE pointers unless marked "host". The caller owns
 *              every buffer (inputs, outputs, workspace); the library never
 *              allocates device memory and keeps no mutable global state.
 * Streams.     `stream` is a hipStream_t (NULL = the default stream). All work
 *              is enqueued on it; outputs are valid once the stream reaches them.
 * Workspace.   Each entry point has a *_workspace_size query; pass at least
 *              that many bytes, 256-byte aligned. Contents need no initialising.
 * Errors.      Every argument is checked on the host before anything is
 *              launched; on error nothing is written and nothing is launched,
 *              and rlk_last_error() (thread-local) holds a message.
 *              Per-row data conditions are not errors: they set flag bits.
 * Determinism. Results are bitwise identical run to run. Per-row outputs do
 *              not depend on the number of rows, their order, or the row
 *              stride (reductions run in a fixed order fixed by the vocabulary
 *              size alone: Qwen3-8B VIME train-rollout consistency page,
 *              "Canonical topology strategy", combines vocabulary shards in one
 *              fixed order so that reduction boundaries never move).
 * Reentrancy.  Concurrent calls on different streams with distinct workspaces
 *              and outputs are safe.
 * Parameters.  Temperature must be finite and > 0 (temperature 0 is
 *              rejected rather than ignored: consistency page, "ROCm MI300X
 *              and gfx942"); top-p must lie in (0, 1]; top-k >= 0, where 0
 *              (the default) means no top-k. Top-k is opt-in: the
 *              consistency page's strict replay contract rejects it, while the
 *              prime-rl v0.10.0 release notes ("2. RL Algorithms") replay a
 *              top-k sampler exactly in the trainer; the sampler and every
 *              scorer here apply the same rule, so the replay stays exact.
 * Top-k rule.  Temperature first; then S_k = {i : z_i >= v_k}, v_k the k-th
 *              largest finite logit (ties with it are all kept, so |S_k| >= k;
 *              k at or above the number of finite logits keeps them all);
 *              then the top-p rule on the distribution renormalised over S_k.
 *              At top-p 1 the nucleus is S_k and its threshold is v_k.
 */
#ifndef RLK_H
#define RLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rlk_status;
#define RLK_OK 0
#define RLK_EINVAL 1        /* bad argument value, shape, stride or pointer */
#define RLK_EUNSUPPORTED 2  /* a valid but unsupported request (reserved) */
#define RLK_EWORKSPACE 3    /* workspace missing, misaligned or too small */
#define RLK_EHIP 4          /* a HIP runtime call failed */

/* logits dtypes */
#define RLK_DTYPE_F32 0
#define RLK_DTYPE_BF16 1

/* per-row flag bits (uint8) */
#define RLK_FLAG_OUTSIDE 1u     /* target outside the nucleus: truncated logprob = -inf */
#define RLK_FLAG_BAD_TARGET 2u  /* target id outside [0, V): logprobs NaN */
#define RLK_FLAG_NONFINITE 4u   /* a NaN / +inf logit, or no finite logit: outputs NaN */
#define RLK_FLAG_BOUNDARY 8u    /* nucleus mass within 1e-6 of top-p (advisory) */
#define RLK_FLAG_BAD_PARAM 16u  /* per-row temperature or top-p out of range: outputs NaN */
#define RLK_FLAG_BAD_SUPPORT 32u /* retained-support scoring: the row's set is empty, out of
                                    range or not strictly increasing: outputs NaN */
#define RLK_FLAG_MISMATCH 64u   /* retained-support scoring with a top-p check: the set is not
                                    the nucleus recomputed from the logits */

/* ABI version of this header: 2. */
int32_t rlk_abi_version(void);

/* Static text for a status code. */
const char* rlk_status_str(rlk_status status);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* rlk_last_error(void);

/* --------------------------------------------------------------------------
 * Logits in: full and top-p truncated log-probability and entropy per row.
 *
 * Consistency page, "ROCm MI300X and gfx942": temperature and top-p are user
 * parameters, the complete retained (nucleus) token set is scored with no
 * support cap, top-p = 1 uses the full vocabulary, and a "monitoring entropy"
 * is fused with the logprob. RL-Kernel ROCm sparse performance page,
 * quick-start command: temperature 0.7, top-p 0.95. Per-row top-p is part of
 * that page's test suite (last paragraphs).
 *
 * For row n with logits z[0..V), target y = targets[n], T, p:
 *   d_i = (z_i - max z) / T;  Z = sum exp(d_i)
 *   lp_full[n]       = d_y - log Z
 *   entropy_full[n]  = log Z - sum exp(d_i) d_i / Z
 *   nucleus S        = {i : z_i >= tau}, tau the lowest row value whose
 *                      strictly-higher mass is < p (so the token crossing p
 *                      and every token tied with it are kept); p = 1 keeps all
 *                      finite tokens and reports tau = -inf
 *   lp_trunc[n]      = d_y - log sum_{i in S} exp(d_i), or -inf if y not in S
 *   entropy_trunc[n] = entropy of the distribution renormalised over S
 *
 * logits        [n_rows, row_stride] fp32 or bf16 (dtype); only the first
 *               `vocab` entries of each row are read (padded vocabularies).
 *               -inf entries are allowed (probability 0).
 * targets       [n_rows] int64 target ids.
 * temperature, top_p, top_k   scalars used for every row, unless the per-row
 *               arrays temperature_per_row / top_p_per_row ([n_rows] fp32) /
 *               top_k_per_row ([n_rows] int32), each nullable, are given;
 *               per-row values out of range (a negative k included) set
 *               RLK_FLAG_BAD_PARAM and NaN outputs. top_k: see "Top-k rule"
 *               above (0: none); the nucleus S below is then the top-k set's.
 * lp_full, lp_trunc, entropy_trunc   [n_rows] fp32 outputs (required).
 * entropy_full  [n_rows] fp32 (nullable).
 * nucleus_size  [n_rows] int32 |S| (nullable).
 * threshold     [n_rows] fp32 tau, the smallest kept logit value (nullable).
 * flags         [n_rows] uint8 RLK_FLAG_* (nullable).
 * Limits: 1 <= vocab <= 2^24, row_stride >= vocab, n_rows >= 0 (0 is a no-op),
 * logits and outputs naturally aligned.
 * -------------------------------------------------------------------------- */
size_t rlk_logprob_from_logits_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype);

rlk_status rlk_logprob_from_logits(
    const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab, int64_t row_stride,
    const int64_t* targets, float temperature, float top_p,
    const float* temperature_per_row, const float* top_p_per_row, int32_t top_k,
    const int32_t* top_k_per_row,
    float* lp_full, float* lp_trunc, float* entropy_trunc,
    float* entropy_full, int32_t* nucleus_size, float* threshold, uint8_t* flags,
    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Logits in, without allocating: rlk_logprob_from_logits for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, outputs and results as rlk_logprob_from_logits (bitwise),
 * without workspace and workspace_bytes. Its scratch (the per-row hand-off
 * flags of the bf16 row kernel and, with top-k, each row's top-k floor, all
 * written for every row before they are read, so nothing needs clearing) is a
 * static 5 MiB device array in the library:
 * each GPU the library runs on holds its own copy until the process ends,
 * its address looked up once per device on the first call there. This call
 * allocates nothing and calls no allocating routine.
 * Limits: n_rows <= 2^20 (RLK_EINVAL above that, before anything is launched),
 * otherwise as rlk_logprob_from_logits.
 * Concurrency: every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (e.g. on two streams) race and must be serialised by the
 * caller; calls on different GPUs are independent.
 * -------------------------------------------------------------------------- */
rlk_status rlk_logprob_from_logits_noalloc(
    const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab, int64_t row_stride,
    const int64_t* targets, float temperature, float top_p,
    const float* temperature_per_row, const float* top_p_per_row, int32_t top_k,
    const int32_t* top_k_per_row,
    float* lp_full, float* lp_trunc, float* entropy_trunc,
    float* entropy_full, int32_t* nucleus_size, float* threshold, uint8_t* flags,
    void* stream);

/* --------------------------------------------------------------------------
 * Logits in, retained support: log-probability and entropy over a
 * caller-supplied token set per row.
 *
 * Consistency page, "ROCm MI300X and gfx942": below top-p 1 the rollout
 * sampler hands its complete finite retained-token set to the deterministic
 * logprob kernel, which scores the selected token and the monitoring entropy
 * over that set (the sparse path); prime-rl v0.10.0 release notes,
 * "Breaking changes": the sampling mask travels in CSR form.
 *
 * For row n with S = support_ids[support_offsets[n] .. support_offsets[n+1]):
 *   d_i = (z_i - max_{j in S} z_j) / T,  Z_S = sum_{i in S} exp(d_i)
 *   logprob[n] = d_y - log Z_S, or -inf with RLK_FLAG_OUTSIDE if y is not in S
 *   entropy[n] = log Z_S - sum_{i in S} exp(d_i) d_i / Z_S
 * logits, dtype, n_rows, vocab, row_stride, targets, temperature   as for
 *               rlk_logprob_from_logits.
 * support_offsets  [n_rows + 1] int64 (device): row n's ids are entries
 *               support_offsets[n] .. support_offsets[n+1] - 1 of support_ids.
 * support_ids   [n_support] int32 (device) token ids; a row's ids must be
 *               strictly increasing, in [0, vocab), non-empty and name finite
 *               logits, else the row gets NaN outputs and RLK_FLAG_BAD_SUPPORT
 *               (or RLK_FLAG_NONFINITE). Offsets outside [0, n_support] make
 *               the row invalid; nothing past n_support is read.
 * check_top_p   0: no check. In (0, 1]: each row's nucleus at (temperature,
 *               check_top_p, check_top_k) is recomputed from the logits as by
 *               rlk_logprob_from_logits, and RLK_FLAG_MISMATCH marks a set that
 *               differs from it (RLK_FLAG_BOUNDARY: the row lies within 1e-6 of
 *               the top-p boundary, where another set is equally valid).
 * check_top_k   the top-k of that nucleus (0: none; > 0 needs check_top_p).
 * logprob, entropy [n_rows] fp32 outputs (required); flags [n_rows] uint8
 *               (nullable). Outputs of a row depend on that row only.
 * Workspace: none without the check; with it, the nucleus outputs of every row
 * and the logits-in workspace.
 * -------------------------------------------------------------------------- */
size_t rlk_logprob_from_support_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype,
                                                float check_top_p);

rlk_status rlk_logprob_from_support(
    const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab, int64_t row_stride,
    const int64_t* targets, float temperature,
    const int64_t* support_offsets, const int32_t* support_ids, int64_t n_support,
    float check_top_p, int32_t check_top_k, float* logprob, float* entropy, uint8_t* flags,
    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Top-p sampler on the same row kernel (rollout side of the replay).
 *
 * prime-rl v0.10.0 release notes, "2. RL Algorithms": top-p sampling is
 * replayed exactly in the trainer; consistency page: rollout and training
 * logprobs must agree bitwise. Per row: the nucleus S at (temperature, top_p,
 * top_k), scalars or per-row arrays, as rlk_logprob_from_logits finds it
 * (a row with an out-of-range parameter draws -1 with RLK_FLAG_BAD_PARAM), then
 *   samples[n] = argmax_{i in S} z_i / T - log(-log u_i)   (fp64; the lowest
 *                id on an exact tie; -1 for a row without a finite logit or
 *                with a NaN / +inf one)
 * with u_i = (w + 1/2) 2^-32, w = word i % 4 of Philox-4x32-10 (Salmon et
 * al., SC 2011) on counter (i / 4, key_n low 32 bits, key_n high 32 bits,
 * offset) and key (seed low 32 bits, seed high 32 bits); key_n = row_keys[n]
 * (nullable: n). A draw depends on its row, seed, offset and key only.
 * logprob, entropy, nucleus_size, flags (nullable): the drawn token scored as
 * rlk_logprob_from_logits scores a target (the row kernel's own row max and
 * log Z_S, the same fp64 arithmetic; entropy, size and flags from the same
 * pass), so they equal bitwise what a training-side call with
 * targets = samples (and the same temperature, top-p and top-k) returns.
 * Limits: as rlk_logprob_from_logits; n_rows < 2^31.
 * -------------------------------------------------------------------------- */
size_t rlk_sample_top_p_workspace_size(int64_t n_rows, int64_t vocab, int32_t dtype);

rlk_status rlk_sample_top_p(
    const void* logits, int32_t dtype, int64_t n_rows, int64_t vocab, int64_t row_stride,
    float temperature, float top_p, int32_t top_k, const float* temperature_per_row,
    const float* top_p_per_row, const int32_t* top_k_per_row,
    uint64_t seed, uint32_t offset, const int64_t* row_keys,
    int64_t* samples, float* logprob, float* entropy, int32_t* nucleus_size, uint8_t* flags,
    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Fused LM head, forward: logprob and entropy of targets under softmax(h W^T / T)
 * without materialising the [N, V] logits (prime-rl v0.10.0 release notes,
 * "1. Trainer Performance": the loss is chunked torchtitan-style).
 *
 * hidden        [n_rows, h_stride] bf16, first hidden_size entries used.
 * weight        [vocab, w_stride] bf16 LM-head rows, first hidden_size used.
 * targets       [n_rows] int64.
 * Logits are accumulated in fp32 over the hidden dimension and never rounded
 * to bf16. With top_p < 1 or top_k > 0 the outputs are the truncated ones of
 * the logits-in entry point (same nucleus rule; the fp32 logits of up to
 * 16384 rows at a time are formed in the workspace and cut by the logits-in
 * row kernel); otherwise they are full and no logits are stored.
 * logprob, entropy   [n_rows] fp32 outputs (required).
 * saved         [n_rows, 4] fp32 (nullable): (log Z_S and E_q[z/T] over the
 *               nucleus, both on the scale z/T; tau, the smallest kept logit,
 *               -inf without a cut; 1 when the row's logprob term is live -- target
 *               in range and kept -- else 0), consumed by
 *               rlk_logprob_fused_linear_bwd.
 * nucleus_size  [n_rows] int32 (nullable).  flags [n_rows] uint8 (nullable):
 *               RLK_FLAG_NONFINITE with NaN outputs for a row with a NaN or
 *               infinite logit (e.g. from a non-finite hidden or weight value).
 * Limits: hidden_size % 64 == 0, 1 <= vocab <= 2^24, 0 <= n_rows < 2^23,
 * strides >= hidden_size, multiples of 8 and < 2^23, hidden/weight 16-byte
 * aligned.
 * -------------------------------------------------------------------------- */
size_t rlk_logprob_fused_linear_workspace_size(int64_t n_rows, int64_t hidden_size,
                                                int64_t vocab, float top_p, int32_t top_k);

rlk_status rlk_logprob_fused_linear(
    const void* hidden, const void* weight, int64_t n_rows, int64_t hidden_size, int64_t vocab,
    int64_t h_stride, int64_t w_stride, const int64_t* targets,
    float temperature, float top_p, int32_t top_k,
    float* logprob, float* entropy, float* saved, int32_t* nucleus_size, uint8_t* flags,
    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Fused LM head, backward by chunk recompute.
 *
 * Given per-row upstream gradients g_lp = dL/dlogprob and g_H = dL/dentropy
 * (already divided by the token count: the loss seed is normalised before
 * model derivatives, consistency page, "Canonical topology strategy"), with
 * q the renormalised distribution on the nucleus S recorded in `saved`:
 *   G[n,i] = (1/T) [ g_lp (delta_{i,y} - q_i) - g_H q_i (z_i/T - E_q[z/T]) ] on S, 0 off S
 *   grad_hidden = G W   (bf16 out, fp32 accumulate)
 *   grad_weight = G^T h (fp32 out, overwritten)
 * The nucleus is the forward's, held fixed (the cut is not differentiated):
 * S = {i : z_i >= tau} with tau from `saved`, the recomputed fp32 logits being
 * summed over the hidden dimension in the forward's order. A row whose target
 * is outside S (or out of range) contributes only its entropy term.
 * grad_logprob, grad_entropy  [n_rows] fp32 (nullable = zeros).
 * saved         [n_rows, 4] fp32 from the forward call with the same inputs.
 * grad_hidden   [n_rows, hidden_size] bf16, dense (required when n_rows > 0).
 * grad_weight   [vocab, hidden_size] fp32, dense (required; zeros when n_rows = 0).
 * The vocabulary is processed in chunks of 32768 rows in a fixed order (so a
 * row of grad_hidden does not depend on the other rows); the workspace holds
 * W^T and h^T (bf16, padded to multiples of 64), G of one chunk in both
 * orientations (bf16) and, when vocab > 32768, an fp32 [n_rows, hidden_size]
 * partial sum of grad_hidden.
 * temperature, top_p and top_k must be the forward call's (top_p and top_k are
 * validated; the nucleus itself comes from `saved`).
 * Limits: as the forward, and vocab < 2^23.
 * -------------------------------------------------------------------------- */
size_t rlk_logprob_fused_linear_bwd_workspace_size(int64_t n_rows, int64_t hidden_size,
                                                    int64_t vocab, float top_p);

rlk_status rlk_logprob_fused_linear_bwd(
    const void* hidden, const void* weight, int64_t n_rows, int64_t hidden_size, int64_t vocab,
    int64_t h_stride, int64_t w_stride, const int64_t* targets, const float* saved,
    const float* grad_logprob, const float* grad_entropy,
    float temperature, float top_p, int32_t top_k,
    void* grad_hidden, float* grad_weight,
    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * GRPO / DAPO token loss over a packed ragged batch.
 * (Every input lives in device memory, so a call can be captured in a HIP graph.)
 *
 * LumenRL README, "Key Features" (GRPO, DAPO, PPO) and "Rollout Correction"
 * (TIS clips large ratios); RL-Kernel ROCm sparse performance page: KL
 * coefficient 0.01 (quick-start command), GRPO standard-deviation
 * normalisation and eight samples per prompt (profile paragraph).
 * For response j (group g = j / group_size) and its tokens t:
 *   A_j    = (r_j - mean_g r) / (std_g r + adv_eps)      (rewards given), or
 *   A_j    = advantages[j]                               (advantages given)
 *   rho    = exp(lp_new - lp_old),  rho~ = min(rho, tis_cap)
 *   s      = min(rho~ A, clip(rho~, 1 - eps_low, 1 + eps_high) A)
 *   k3     = exp(lp_ref - lp_new) - (lp_ref - lp_new) - 1
 *   l_t    = -s + kl_coef k3;   loss = sum_t l_t / T_tot  (token mean)
 *   dL/dlp_new = (-A rho [rho <= C, clip not binding] + kl_coef (1 - exp(lp_ref - lp_new))) / T_tot
 * lp_new, lp_old, lp_ref  [T_tot] fp32 (lp_ref nullable when kl_coef == 0).
 * cu_seqlens    [n_seqs + 1] int64 packed offsets (device), which must be
 *               non-decreasing from 0 to n_tokens. They are checked on the
 *               device: invalid offsets make loss, grad_lp_new, token_loss,
 *               metrics and adv_out NaN (token_flags 0) and set *status = 1.
 * n_tokens      T_tot, the packed token count (by value).
 * rewards / advantages    [n_seqs] fp32: exactly one must be non-NULL.
 * group_size    responses per prompt; must divide n_seqs (rewards mode).
 * (The variants of rlk_grpo_params below change s, rho~, the baseline and the
 * token weights; the defaults are the formulas above.)
 * loss          device fp32 scalar (required).  grad_lp_new [T_tot] fp32 (required).
 * token_loss    [T_tot] fp32 (nullable).  token_flags [T_tot] uint8 (nullable):
 *               bit0 TIS cap binds (rho > C), bit1 clipped branch taken.
 * metrics       [4] fp32 (nullable): token means of clip flag, TIS flag, k3, rho.
 * adv_out       [n_seqs] fp32 (nullable): the advantages used. A group whose
 *               rewards are all equal gets A = 0 exactly in every mode.
 * status        device int32 (nullable): 0 when cu_seqlens was valid, else 1.
 * T_tot == 0 gives loss 0. Limits: 1 <= n_seqs <= 2^31, 0 <= n_tokens <= 2^40.
 * -------------------------------------------------------------------------- */
/* Loss variants (prime-rl v0.10.0 release notes, "2. RL Algorithms": IPO
 * masks a token when |pi_train - pi_infer| > eps (eps 0.3, no KL term);
 * IcePop masks it when pi_train / pi_infer leaves a fixed band; CISPO stays an
 * opt-in loss; GRPO gains a length-weighted baseline and exact prompt-mean
 * aggregation. "Breaking changes": zero-advantage samples are filtered.
 * LumenRL README, "Rollout Correction": MIS normalises the ratios.)
 * pi_infer = exp(lp_old), pi_train = exp(lp_new); rho~ per `correction`:
 *   TIS: rho~ = min(rho, tis_cap);  MIS: rho~ = rho / mean(rho) over the
 *   tokens entering the loss (the mean held constant).
 *   DAPO:   s = min(rho~ A, clip(rho~, 1 - eps_low, 1 + eps_high) A)   (above)
 *   IPO:    s = [|exp(lp_new) - exp(lp_old)| <= ipo_eps] rho~ A
 *   ICEPOP: s = [icepop_lo <= rho <= icepop_hi] rho~ A
 *   CISPO:  s = w A lp_new, w = clip(rho~, 1 - eps_low, 1 + eps_high) held
 *           constant (gradient -w A)
 *   TIS_PG: the detached-TIS form: rho~ a constant weight on an on-policy
 *           surrogate (its ratio is 1 at the evaluation point): s = rho~ A,
 *           gradient -rho~ A, no clip
 * Token flag bit1 marks the clipped branch (DAPO), a masked token (IPO,
 * ICEPOP) or a binding clip on w (CISPO); metrics[0] is its token mean.
 * baseline LENGTH (rewards mode): the group baseline is sum_j L_j r_j /
 * sum_j L_j with L_j the response's token count. filter_zero_adv: a response
 * with A_j == 0 is left out of the loss and of the counts. aggregation
 * PROMPT_MEAN: a kept token of group g (group_size consecutive responses,
 * in both modes) weighs 1 / (G_kept T_g), T_g the kept tokens of group g and
 * G_kept the groups with T_g > 0; TOKEN_MEAN: 1 / T_kept. The loss is the
 * weighted sum of l_t and dL/dlp_new carries the same weight. */
#define RLK_LOSS_DAPO 0
#define RLK_LOSS_IPO 1
#define RLK_LOSS_ICEPOP 2
#define RLK_LOSS_CISPO 3
#define RLK_LOSS_TIS_PG 4
#define RLK_CORRECTION_TIS 0
#define RLK_CORRECTION_MIS 1
#define RLK_AGG_TOKEN_MEAN 0
#define RLK_AGG_PROMPT_MEAN 1
#define RLK_BASELINE_MEAN 0
#define RLK_BASELINE_LENGTH 1

typedef struct rlk_grpo_params {
    uint32_t struct_size;   /* sizeof(rlk_grpo_params); the first layout (up to
                               normalize_std, 32 bytes) is accepted and takes the
                               defaults for the fields after it */
    float tis_cap;          /* C > 0, e.g. 2.0 */
    float eps_low;          /* in [0, 1), e.g. 0.2 */
    float eps_high;         /* >= 0, e.g. 0.28 */
    float kl_coef;          /* >= 0, e.g. 0.01 */
    float adv_eps;          /* >= 0, e.g. 1e-6 */
    int32_t std_ddof;       /* 0 or 1 */
    int32_t normalize_std;  /* 1 = divide by the group std */
    int32_t loss_type;      /* RLK_LOSS_* (default DAPO) */
    int32_t correction;     /* RLK_CORRECTION_* (default TIS) */
    int32_t aggregation;    /* RLK_AGG_* (default TOKEN_MEAN) */
    int32_t filter_zero_adv;/* 0 or 1 (default 0) */
    int32_t baseline;       /* RLK_BASELINE_* (default MEAN) */
    float ipo_eps;          /* > 0 (default 0.3) */
    float icepop_lo;        /* 0 < icepop_lo <= icepop_hi (defaults 0.5, 2.0) */
    float icepop_hi;
} rlk_grpo_params;

size_t rlk_grpo_token_loss_workspace_size(int64_t n_tokens, int64_t n_seqs);

rlk_status rlk_grpo_token_loss(
    const float* lp_new, const float* lp_old, const float* lp_ref,
    const int64_t* cu_seqlens, int64_t n_seqs, int64_t n_tokens,
    const float* rewards, const float* advantages, int32_t group_size,
    const rlk_grpo_params* params,
    float* loss, float* grad_lp_new, float* token_loss, uint8_t* token_flags,
    float* metrics, float* adv_out, int32_t* status,
    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H */
