// Types shared between the self-conditioning kernels and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

// GEMM tiling of the self-conditioning product: workgroups of 8 waves, each
// computing a kSelfCondTileM x kSelfCondTileN tile of out over one of
// kSelfCondSplits vocab ranges. d is a multiple of kSelfCondDMultiple; the
// last column tile may be half full.
constexpr int kSelfCondThreads = 512;
constexpr int kSelfCondTileM = 128;
constexpr int kSelfCondTileN = 512;
constexpr int kSelfCondDMultiple = 256;
constexpr int kSelfCondSplits = 8;
constexpr int kSelfCondStepK = 32;

struct SelfCondParams {
  const float *logits;
  int64_t ld;
  int64_t rows;
  int32_t vocab;
  int32_t d;            // columns of E and out, a multiple of kSelfCondDMultiple
  const float *temps;
  uint32_t slot_mul;    // row / canvas_len = (row * slot_mul) >> slot_shift
  uint32_t slot_shift;
  const uint64_t *rowres;  // [rows] row results {m, 1 / S} of the row-statistics kernel
  const uint16_t *E;       // bf16 or fp16 (f16) [vocab, d], 16-byte aligned
  float *partial;          // [kSelfCondSplits, rows, d] fp32 scratch
  float *out;              // [rows, d] fp32, 16-byte aligned
  int32_t k_per_split;     // vocab columns of one range, a multiple of kSelfCondStepK
  int32_t m_tiles;
  int32_t n_tiles;
  int32_t vec_ok;          // logits 16-byte aligned and ld % 4 == 0
  int32_t f16;             // model dtype fp16 (else bf16): probabilities and E
};

// Queues the GEMM over all ranges and the fixed-order sum of the partials.
hipError_t selfcond_launch(const SelfCondParams &p, hipStream_t stream);

// Queues out = the sum of kSelfCondSplits partial [rows, d] fp32 products
// (consecutive, rows * d apart), added in range order; d % 4 == 0, partial
// and out 16-byte aligned.
hipError_t partial_sum_launch(const float *partial, int64_t rows, int32_t d, float *out,
                              hipStream_t stream);

}  // namespace rowstats
