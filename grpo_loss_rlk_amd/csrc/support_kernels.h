// Internal launch interface of the retained-support scorer (support.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

struct SupportArgs {
  const void* logits;
  int64_t n_rows, vocab, row_stride;
  const int64_t* targets;
  float temperature;
  const int64_t* offsets;     // [n_rows + 1] CSR row offsets into ids
  const int32_t* ids;         // [n_support] token ids
  int64_t n_support;          // entries of ids (offsets past it make a row invalid)
  float* lp;
  float* ent;
  uint8_t* flags;             // nullable
  // nucleus of the same rows at the checked top-p (all null: no check)
  const int32_t* nsize;
  const float* thresh;
  const uint8_t* nflags;
};

// dtype: 0 = fp32, 1 = bf16
hipError_t launch_support_rows(const SupportArgs& a, int dtype, hipStream_t stream);

}  // namespace rlk
