// Types shared between the top-K logprob kernel and the C ABI of librowstats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

constexpr int kTopKThreads = 512;
constexpr int kTopKQPT = 8;     // quads per thread: slices of 16384 columns
constexpr int kTopKMax = 64;    // largest K served

struct TopKParams {
  const float *logits;
  int64_t ld;
  int64_t rows;
  int32_t vocab;
  int32_t G;
  int32_t nq;
  int32_t nq_full;
  int32_t vec_ok;     // logits 16-byte aligned, ld % 4 == 0, vocab % 4 == 0
  int32_t xcd_map;
  int32_t K;
  const float *temps;
  int64_t canvas_len;
  const uint8_t *keep;
  float *out_vals;
  int64_t *out_idx;
  void *partials;       // [rows, G] records of topk_partial_bytes(K)
  uint32_t *counters;   // two banks of counter_stride words, alternated by call
  int64_t counter_stride;
  int32_t parity;       // bank this call counts in
};

// Per-slice record: double S, float m, pad, then K 64-bit keys.
__host__ __device__ inline size_t topk_partial_bytes(int K) {
  return (16 + 8 * (size_t)K + 15) & ~(size_t)15;
}

hipError_t topk_resident_blocks(bool vec, int *blocks_per_cu);
hipError_t topk_launch(const TopKParams &p, int grid, hipStream_t stream);

}  // namespace rowstats
