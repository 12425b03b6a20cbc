// Types shared between the top-K logprob kernels and the C ABI of librowstats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rowstats_internal.h"

namespace rowstats {

constexpr int kTopKMax = 64;  // largest K served

// Per (kept row, chunk) record in global scratch: a header of two tagged
// words (chunk maximum m, S = sum exp(s - m)) and the chunk's K largest
// keys in rank order, each as two tagged words (high, low half). Every
// word carries the call's epoch in its high half.
__host__ __device__ inline size_t topk_record_bytes(int K) { return 16 * ((size_t)K + 1); }

struct TopKParams {
  const float *logits;
  int64_t ld;
  int64_t rows;
  int32_t vocab;
  int32_t C;          // chunks per row, ceil(vocab / kChunkCols): the waves of a group
  int32_t n_groups;   // groups, each reducing kept rows group, group + n_groups, ...
  int32_t vec_ok;     // logits 16-byte aligned, ld % 4 == 0, vocab % 4 == 0
  int32_t K;
  uint32_t epoch;     // tag of this call's scratch words (never 0)
  const float *temps;
  int64_t canvas_len;
  const uint8_t *keep;
  float *out_vals;
  int64_t *out_idx;
  int64_t *kept;      // [rows + 1]: kept rows in order, then their count (written by the pre-pass)
  float *kept_temp;   // [rows]: temperature of kept row i (written by the pre-pass)
  uint64_t *records;  // [rows, C] records of topk_record_bytes(K), indexed by kept position
  uint64_t *rowres;   // [rows] row results of kRowResultBytes, indexed by kept position
  uint64_t *rings;    // [n_groups] rings of kept positions (RowDealer)
  uint32_t *counters; // two row-claim counters: a call uses counters[epoch & 1]
                      // (the pre-pass zeroes both)
  uint32_t *err_flag;  // the scratch's error words: {report bits, failed epoch}

  // Stash mode (stash != 0): rows come from requests instead of slots and
  // each kept row is written as one stash row.
  int32_t stash;
  int32_t K_out;         // top-K columns of a stash row (K above is max(K_out, 2), capped at vocab)
  int32_t logits_mode;   // write s instead of s - log Z
  int32_t width;         // stash row width, >= K_out + 1
  int64_t m;             // requests
  int64_t logits_rows;   // rows of the logits matrix
  int64_t stash_slots;   // first dimension of the stash
  int64_t positions;     // second dimension of the stash (>= canvas_len)
  const int32_t *src;    // [m] canvas of request j
  const int32_t *slots;  // [m] stash slot of request j
  const int32_t *valid;  // [m] positions of request j
  const int32_t *num_ids;  // [m] token ids of request j (null: none)
  const int32_t *ids;      // [m, ids_stride]
  int64_t ids_stride;
  int32_t *out_ids32;    // [stash_slots, positions, width]
  float *out_lp;         // [stash_slots, positions, width]
  int32_t *out_ranks;    // [stash_slots, positions]
  int64_t *kept_dst;     // [rows]: stash row slots[j] * positions + p of kept row i
  int32_t *kept_req;     // [rows]: request j of kept row i
};

hipError_t topk_resident_blocks(bool vec, int *blocks_per_cu);
// Queues the kept-row pre-pass and the top-K kernel (cooperative) on `stream`.
hipError_t topk_launch(const TopKParams &p, int grid, hipStream_t stream);
// Queues the kept-row pre-pass alone (p.keep, p.temps, p.rows, p.canvas_len,
// p.kept, p.kept_temp, p.counters).
hipError_t kept_rows_launch(const TopKParams &p, hipStream_t stream);
// Queues the stash's kept-row pre-pass alone (the stash fields, p.kept,
// p.kept_temp, p.kept_dst, p.kept_req, p.counters, p.err_flag).
hipError_t stash_rows_launch(const TopKParams &p, hipStream_t stream);
// K > kTopKMax (up to the vocabulary), or a stash with K_out > kTopKMax: the
// kept-row pre-pass and one workgroup per kept position (p.rows of them, the
// surplus returns at once); uses p.logits, p.ld, p.vocab, p.vec_ok, p.K,
// p.out_vals, p.out_idx (or the stash fields) and the pre-pass outputs.
hipError_t topk_wide_launch(const TopKParams &p, hipStream_t stream);

}  // namespace rowstats
