// Types shared between the probabilities x packed-embedding product kernels
// and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

// GEMM tiling: workgroups of 8 waves, each computing a kProductTileM x
// kProductTileN tile of out over one of kProductSplits vocab ranges, in steps
// of kProductStepK vocab rows. d is a multiple of kProductDMultiple; the last
// column tile may be half full.
constexpr int kProductThreads = 512;
constexpr int kProductTileM = 128;
constexpr int kProductTileN = 512;
constexpr int kProductStepK = 64;
constexpr int kProductSplits = 8;
constexpr int kProductDMultiple = 256;
// The packed table holds ceil(vocab / kPackRows) * kPackRows vocab rows (the
// rows past vocab are zero), in blocks of kPackBlock x kPackBlock elements.
constexpr int kPackRows = 128;
constexpr int kPackBlock = 32;

// Bytes of the packed table of a [vocab, d] embedding (2-byte elements).
inline int64_t packed_embed_bytes(int64_t vocab, int64_t d) {
  return (vocab + kPackRows - 1) / kPackRows * kPackRows * d * 2;
}

struct ProductParams {
  const uint16_t *P;        // [rows, ldp] probabilities, bf16 or fp16
  int64_t ldp;
  int64_t rows;
  int32_t vocab;
  int32_t d;                // a multiple of kProductDMultiple
  const uint16_t *packed;   // packed table, 16-byte aligned
  float *partial;           // [kProductSplits, rows, d] fp32 scratch
  float *out;               // [rows, d] fp32, 16-byte aligned
  int32_t k_per_split;      // vocab rows of one range, a multiple of kProductStepK
  int32_t m_tiles;
  int32_t n_tiles;
  int32_t vec_ok;           // P 16-byte aligned and ldp % 8 == 0
  int32_t f16;              // fp16 (else bf16)
};

// Queues the packing of E [vocab, d] (row-major, 2-byte elements) into
// `packed` (packed_embed_bytes(vocab, d) bytes).
hipError_t pack_embed_launch(const uint16_t *E, int64_t vocab, int64_t d, uint16_t *packed,
                             hipStream_t stream);

// Queues the GEMM over all ranges and the fixed-order sum of the partials.
hipError_t product_launch(const ProductParams &p, hipStream_t stream);

}  // namespace rowstats
