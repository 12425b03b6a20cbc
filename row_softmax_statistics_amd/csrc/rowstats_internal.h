// Types shared between the kernels and the C ABI of librowstats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

// Row-statistics work split: a row is cut into chunks of kChunkCols columns;
// one wave reduces one chunk at a time, each lane holding kWaveQuads quads
// (4 columns) in registers. Workgroups of kRowThreads threads only group
// waves for launch and LDS; waves exchange results through global scratch.
constexpr int kWaveQuads = 8;
constexpr int kRowThreads = 256;
constexpr int kChunkQuads = 64 * kWaveQuads;  // 512
constexpr int kChunkCols = 4 * kChunkQuads;   // 2048

// Global scratch per (row, member wave): eight tagged 64-bit words.
constexpr int kTupleBytes = 64;
// Per row: two tagged words (row maximum, 1 / sum) read by the probs writers.
constexpr int kRowResultBytes = 16;

// Dynamic row assignment (RowDealer): rows claimed this many rows ahead,
// and a ring of this many 16-byte slots per group.
constexpr int kDealAhead = 8;
constexpr int kRingSlots = 16;
constexpr int kRingBytes = 16 * kRingSlots;

// Report bits of a scratch area's first error word: a bounded wait ran out
// (the call's other waits then give up too), and an index argument of the
// stash was out of range (that request or token id is skipped).
constexpr uint32_t kErrWait = 1u;
constexpr uint32_t kErrIndex = 2u;

struct RowStatsParams {
  const float *logits;
  int64_t ld;
  int64_t rows;
  int32_t vocab;
  int32_t C;          // chunks per row, ceil(vocab / kChunkCols): the waves of a group
  int32_t n_groups;   // groups, each reducing rows group, group + n_groups, ...
  int32_t vec_ok;     // 16-byte aligned rows, ld % 4 == 0, vocab % 4 == 0, probs 8-byte aligned
  uint32_t epoch;     // tag of this call's scratch words (never 0)
  const float *temps;
  int64_t canvas_len;
  uint32_t slot_mul;  // row / canvas_len = (row * slot_mul) >> slot_shift for 0 <= row < 2^31
  uint32_t slot_shift;
  uint64_t seed;
  int64_t *argmax;
  int64_t *sample;
  float *entropy;
  void *probs;
  uint64_t *tuples;   // [rows, C] tuples of kTupleBytes
  uint64_t *rowres;   // [rows] row results of kRowResultBytes
  uint64_t *rings;    // [n_groups] rings of rows (RowDealer)
  uint32_t *counters; // two row-claim counters: a call uses counters[epoch & 1]
                      // and zeroes counters[(epoch + 1) & 1] for the next call
  uint32_t *err_flag;  // the scratch's error words: {report bits, failed epoch}
};

// Multiplier and shift with floor(n / d) = (n * mul) >> shift for every
// 0 <= n < 2^31 (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994, with the multiplier rounded up): for
// 2^(l-1) < d <= 2^l, mul = ceil(2^(31 + l) / d) < 2^32 and shift = 31 + l.
// d >= 2^31 maps every such n to 0.
inline void slot_divider(int64_t d, uint32_t *mul, uint32_t *shift) {
  if (d >= 0x80000000LL) {
    *mul = 0;
    *shift = 0;
    return;
  }
  int l = 0;
  while ((int64_t(1) << l) < d) ++l;
  const uint64_t two = uint64_t(1) << (31 + l);
  *mul = (uint32_t)((two + (uint64_t)d - 1) / (uint64_t)d);
  *shift = (uint32_t)(31 + l);
}

hipError_t rowstats_resident_blocks(int probs_dtype, bool vec, int *blocks_per_cu);
hipError_t rowstats_launch(const RowStatsParams &p, int probs_dtype, int grid,
                           hipStream_t stream);

}  // namespace rowstats
