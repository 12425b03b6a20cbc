// Types shared between the kernels and the C ABI of librowstats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

// Quads (4 columns) per thread held in registers by the row-statistics
// kernel; a slice is 512 threads x kQPT quads = 16384 columns.
constexpr int kQPT = 8;
constexpr int kRowThreads = 512;
constexpr int kSliceCols = kRowThreads * kQPT * 4;

// Words of global scratch per slice tuple (see the kernel).
constexpr int kSliceTupleWords = 5;

struct RowStatsParams {
  const float *logits;
  int64_t ld;
  int64_t rows;
  int32_t vocab;
  int32_t G;          // slices per row
  int32_t nq;         // quads per row, ceil(vocab / 4)
  int32_t nq_full;    // quads entirely inside the row, vocab / 4
  int32_t n_groups;   // probs path: rows processed concurrently
  int32_t vec_ok;     // logits and probs aligned, ld % 4 == 0, vocab % 4 == 0
  int32_t xcd_map;    // grid is a multiple of 8 with G | grid / 8
  int32_t l2_sync;    // the workgroups of every row share one XCD (see the kernel)
  const float *temps;
  int64_t canvas_len;
  uint64_t seed;
  int64_t *argmax;
  int64_t *sample;
  float *entropy;
  void *probs;
  uint64_t *partials; // [rows, G] slice tuples of kSliceTupleWords words
  uint32_t *counters; // two banks of counter_stride words (see the kernel)
  int64_t counter_stride;
  int32_t parity;     // bank this call counts in
  uint32_t *err_flag;
};

hipError_t rowstats_resident_blocks(int probs_dtype, bool vec, int *blocks_per_cu);
hipError_t rowstats_launch(const RowStatsParams &p, int probs_dtype, int grid,
                           hipStream_t stream);

}  // namespace rowstats
