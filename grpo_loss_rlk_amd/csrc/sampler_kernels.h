// Internal launch interface of the top-p sampler (sampler.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

struct SampleArgs {
  const void* logits;
  int64_t n_rows, vocab, row_stride;
  float temperature;
  const float* t_row;         // nullable per-row temperature
  uint64_t seed;
  uint32_t offset;
  const int64_t* row_keys;    // nullable: the row index
  const float* thresh;        // [n_rows] nucleus threshold of each row (logit value)
  const uint8_t* nflags;      // [n_rows] flags of the nucleus pass
  const double* score_stats;  // [n_rows, 2] the nucleus pass's row max and log Z_S
  int64_t* samples;           // [n_rows] out
  float* logprob;             // nullable [n_rows] out: the drawn token's truncated logprob
  uint8_t* flags;             // nullable [n_rows] out: the row's flags for the drawn token
};

// dtype: 0 = fp32, 1 = bf16
hipError_t launch_sample_rows(const SampleArgs& a, int dtype, hipStream_t stream);
hipError_t launch_fill_i64(int64_t* p, int64_t n, int64_t v, hipStream_t stream);

}  // namespace rlk
