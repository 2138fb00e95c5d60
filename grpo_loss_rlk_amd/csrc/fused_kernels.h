// Internal launch interfaces of the fused LM-head kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rlk {

struct FusedFwdArgs {
  const uint16_t* h;       // bf16 [N, hs]
  const uint16_t* w;       // bf16 [V, ws]
  int64_t N, H, V, hs, ws;
  const int64_t* targets;  // [N]
  float c2;                // log2(e) / T
  float* logprob;          // [N]
  float* entropy;          // [N]
  float* saved;            // [N, 4] nullable
  int32_t* nsize;          // [N] nullable
  uint8_t* flags;          // [N] nullable
  float4* part;            // workspace: [ceil(V/256), N] tile partials
  float* zy;               // workspace: [N] target logits
  float temperature, top_p;
  int32_t top_k;           // 0: off; > 0 takes the stored-logits path at any top-p
};

// Tokens per row block of the top-p < 1 path: the block's fp32 logits are
// written to a workspace scratch and cut by the logits-in row kernel.
// Tokens per fp32 logits block of the fused forward at top-p < 1: 16384 x
// 151936 fp32 is 10 GB of workspace (small beside 288 GB of HBM); a larger
// block leaves a smaller share of each GEMM launch to its last, partly
// filled round of tiles (32768 tokens: 46.9 ms with 4096-token blocks,
// 46.0 ms with 16384).
constexpr int64_t kTopPRowBlock = 16384;

size_t fused_fwd_workspace(int64_t N, int64_t H, int64_t V, float top_p, int32_t top_k);
hipError_t launch_fused_fwd(FusedFwdArgs a, void* workspace, hipStream_t stream);

struct FusedBwdArgs {
  const uint16_t* h;       // bf16 [N, hs]
  const uint16_t* w;       // bf16 [V, ws]
  int64_t N, H, V, hs, ws;
  const int64_t* targets;  // [N]
  const float* saved;      // [N, 4]: log Z of z/T, E_q[z/T], (cut), (unused)
  const float* g_lp;       // [N] nullable (zeros)
  const float* g_H;        // [N] nullable (zeros)
  float inv_t;             // 1 / T
  uint16_t* dh;            // bf16 [N, H] out
  float* dW;               // fp32 [V, H] out
};

// Vocabulary rows per chunk of the backward: fixed, so that the summation
// order of a row of dh does not depend on the number of rows.
constexpr int64_t kBwdChunk = 32768;

size_t fused_bwd_workspace(int64_t N, int64_t H, int64_t V);
hipError_t launch_fused_bwd(const FusedBwdArgs& a, void* workspace, hipStream_t stream);

}  // namespace rlk
