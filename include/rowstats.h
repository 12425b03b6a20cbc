/*
 * rowstats: one-pass row statistics of temperature-scaled logits and top-K
 * logprobs of converged slots, for the DiffusionGemma denoise sampler
 * (vLLM API page "diffusion_gemma_sampler").
 *
 * C ABI of librowstats.so (HIP, gfx950). Every pointer argument except the
 * stream is DEVICE memory owned by the caller; the library keeps no pointer
 * after a call returns. Work is queued asynchronously on `stream` (a
 * hipStream_t passed as void*, NULL = the default stream): buffers must stay
 * alive until that stream has been synchronised. rowstats_run,
 * rowstats_selfcond, rowstats_selfcond_product, topk_logprobs and
 * stash_converged_logprobs share grow-only scratch buffers per device: a call
 * queued on another stream than the previous one
 * first waits, on the device, for that previous call (an event wait), so
 * calls from several streams run one after another. rowstats_run_noalloc
 * has a fixed scratch array of its own (see there).
 *
 * All functions return ROWSTATS_OK (0) or a negative rowstats_status; they
 * never abort and never throw. Argument checks run before any HIP call, so
 * a rejected call touches neither the device nor the outputs.
 * rowstats_last_error() describes the last failure of the calling thread.
 */
#ifndef ROWSTATS_H
#define ROWSTATS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rowstats_status {
  ROWSTATS_OK = 0,
  ROWSTATS_ERR_NULL = -1,   /* a required pointer is NULL */
  ROWSTATS_ERR_SHAPE = -2,  /* rows < 0, or (rows > 0 and: rows > 2^31 - 1,
                               vocab < 1, vocab > 2^31 - 1 - 65536,
                               row_stride < vocab, canvas_len < 1) */
  ROWSTATS_ERR_K = -3,      /* K < 1 or K > vocab; for the stash num_topk < 0
                               or num_topk > vocab */
  ROWSTATS_ERR_DTYPE = -4,  /* probs_dtype is not one of rowstats_probs_dtype */
  ROWSTATS_ERR_HIP = -5,    /* a HIP call failed (allocation, launch); see last_error */
  ROWSTATS_ERR_COOP = -6,   /* rowstats_run keeps the ceil(vocab / 2048) chunks of a
                               row in co-resident waves at once and the device
                               cannot hold them (vocab above about 4.2 million on
                               one MI355X) */
  ROWSTATS_ERR_DEVICE = -7, /* a kernel flagged a failure (a bounded wait ran out,
                               or a stash index argument was out of range);
                               reported by rowstats_check_device */
  ROWSTATS_ERR_SCRATCH = -8 /* rowstats_run_noalloc: the call needs more scratch
                               than ROWSTATS_NOALLOC_SCRATCH_BYTES */
} rowstats_status;

/* Size of the fixed scratch array of rowstats_run_noalloc (64 MiB per GPU). */
#define ROWSTATS_NOALLOC_SCRATCH_BYTES (64ull << 20)

typedef enum rowstats_probs_dtype {
  ROWSTATS_PROBS_NONE = 0,
  ROWSTATS_PROBS_BF16 = 1,
  ROWSTATS_PROBS_FP16 = 2
} rowstats_probs_dtype;

/*
 * For each row of a [rows, vocab] fp32 logits matrix: the argmax, a
 * Gumbel-max sample and the entropy, and on request the softmax.
 * Defined by: diffusion_gemma_sampler page, module docstring (one read per
 * row, online max and sum, noise drawn inline, probs written once),
 * sample_row_stats (arguments, outputs, the greedy rule) and
 * sample_row_stats_reference (the statistics themselves).
 *
 *   logits      fp32, element (r, c) at logits[r * row_stride + c]; unit
 *               column stride; row_stride >= vocab (padded rows allowed).
 *               Values are finite or -inf; no row is all -inf; x / T stays
 *               finite in fp32 (not checked on the device).
 *   rows, vocab matrix shape; rows == 0 returns at once;
 *               rows <= 2^31 - 1; 1 <= vocab <= 2^31 - 1 - 65536.
 *   temps       fp32, at least ceil(rows / canvas_len) entries; row r uses
 *               T = temps[r / canvas_len]. T > 0 samples with Gumbel noise;
 *               T <= 0 is greedy (sample = argmax). The scaled logits are
 *               s = x / max(T, 1e-10f) (IEEE fp32 division).
 *   canvas_len  rows per temperature slot, >= 1.
 *   seed        noise seed: column c of row r draws word c & 3 of
 *               Philox4x32-10(counter = (c >> 2, 0, lo32(r), hi32(r)),
 *               key = (lo32(seed), hi32(seed))); u = (w + 0.5) 2^-32 and
 *               the Gumbel variate is -log(-log u), scored in fp64.
 *   probs_dtype ROWSTATS_PROBS_NONE, _BF16 or _FP16.
 *   argmax      int64 [rows]: lowest column attaining max_c s (-0 == +0).
 *   sample      int64 [rows]: lowest column attaining max_c s + g (T > 0),
 *               the argmax otherwise.
 *   entropy     fp32 [rows]: -sum_{p>0} p log p of p = softmax(s).
 *   probs       NULL when probs_dtype is NONE, else [rows, vocab] contiguous
 *               (row stride vocab) bf16 or fp16: softmax(s) rounded to
 *               nearest-even, subnormals kept, 0 on -inf columns.
 *   stream      hipStream_t or NULL.
 */
int rowstats_run(const float *logits, int64_t row_stride, int64_t rows,
                 int64_t vocab, const float *temps, int64_t canvas_len,
                 uint64_t seed, int probs_dtype, int64_t *argmax,
                 int64_t *sample, float *entropy, void *probs, void *stream);

/*
 * rowstats_run without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, outputs and errors as
 * rowstats_run, computed by the same kernels; it calls no hipMalloc,
 * hipFree or other allocating routine. Its scratch is a file-scope
 * __device__ array of ROWSTATS_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends. A call needs
 *   256 + G * 256 + rows * ceil(vocab / 2048) * 64 + rows * 16 bytes
 * (G = the row groups of the launch, at most 4096 / ceil(vocab / 2048));
 * more returns ROWSTATS_ERR_SCRATCH before anything is queued. At vocab
 * 262144 that is up to 8000 rows per call.
 * Every call on a GPU shares that GPU's array and leaves its contents for
 * the next one. A call first clears the part of the array it uses with a
 * fill kernel (no memset node), so a call captured into a HIP graph can be
 * replayed any number of times (a replay keeps the epoch its words were
 * tagged with at capture; the clearing keeps an earlier replay's words from
 * passing for its own). Calls of this entry point that overlap in time on
 * one GPU (two streams, two threads, two graphs) race on the array: queue
 * them on one stream.
 */
int rowstats_run_noalloc(const float *logits, int64_t row_stride, int64_t rows,
                         int64_t vocab, const float *temps, int64_t canvas_len,
                         uint64_t seed, int probs_dtype, int64_t *argmax,
                         int64_t *sample, float *entropy, void *probs,
                         void *stream);

/*
 * The row statistics of rowstats_run (without probs) and the
 * self-conditioning input of the denoise step: the softmax of each row in
 * the model dtype (bf16 or fp16) times the token embedding table, computed
 * on the matrix cores without writing the probabilities,
 *   out[r, j] = sum_c q_r[c] * E[c, j],   q_r = dtype(softmax(s_r)),
 * q_r being the probabilities rowstats_run writes with the same probs_dtype
 * (each within one unit of the exact rounding).
 * Defined by: diffusion_gemma_sampler page, module docstring (the step's
 * probabilities, kept in the model's own dtype, are the input of the
 * self-conditioning matrix product); the statistics as for rowstats_run.
 *
 *   logits ... seed, argmax, sample, entropy   as for rowstats_run.
 *   dtype       ROWSTATS_PROBS_BF16 or ROWSTATS_PROBS_FP16: the model dtype,
 *               of the probabilities and of embed.
 *   embed       [vocab, d] row-major in that dtype (row c is token c's
 *               embedding), 16-byte aligned.
 *   d           embedding width: a multiple of 256, 256 <= d <= 2^20.
 *   out         fp32 [rows, d] row-major, 16-byte aligned: fp32 sums of the
 *               products (exact in fp32), added in a fixed order (repeat
 *               calls give the same bits).
 *   Scratch: the grow-only scratch, and a grow-only buffer of 8 partial
 *   [rows, d] fp32 products. Errors as for rowstats_run; ROWSTATS_ERR_DTYPE for another
 *   dtype, ROWSTATS_ERR_SHAPE also for a bad d or alignment.
 */
int rowstats_selfcond(const float *logits, int64_t row_stride, int64_t rows,
                      int64_t vocab, const float *temps, int64_t canvas_len,
                      uint64_t seed, int dtype, const void *embed, int64_t d,
                      int64_t *argmax, int64_t *sample, float *entropy,
                      float *out, void *stream);

/*
 * The self-conditioning input from given probabilities, for callers that
 * keep the probabilities (rowstats_run with probs) and the embedding table
 * in the packed order below: out = P E on the matrix cores, E read straight
 * into matrix-core registers (no pass through LDS), P through LDS.
 * Defined by: diffusion_gemma_sampler page, module docstring (the softmax in
 * the model dtype feeds the self-conditioning matmul).
 *
 * rowstats_packed_embed_bytes: bytes of the packed table of a [vocab, d]
 *   embedding, ceil(vocab / 128) * 128 * d * 2; or ROWSTATS_ERR_SHAPE for a
 *   vocab outside [1, 2^31 - 1 - 65536] or a d that is not a multiple of 256
 *   in [256, 2^20].
 *
 * rowstats_pack_embed: queues the packing of `embed` into `packed`, once per
 *   table (the table is a weight; repeat products reuse the packed copy).
 *   embed       [vocab, d] row-major, 2-byte elements (bf16 or fp16 as
 *               `dtype` says; the packing moves bits only), 2-byte aligned.
 *   packed      rowstats_packed_embed_bytes(vocab, d) bytes, 16-byte
 *               aligned, caller-owned: blocks of 32 vocab rows x 32 columns,
 *               block (b, j) at element (b * d / 32 + j) * 1024; inside it,
 *               element h * 512 + l * 8 + i is E[32 b + 16 h + 8 (l / 32) + i]
 *               [32 j + l % 32] (h < 2, l < 64, i < 8), 0 past the last row.
 *   Errors: ROWSTATS_ERR_SHAPE (shape, alignment), _DTYPE, _NULL, _HIP.
 *
 * rowstats_selfcond_product:
 *   probs       [rows, vocab] probabilities in `dtype`, element (r, c) at
 *               probs[r * probs_stride + c], probs_stride >= vocab; 2-byte
 *               aligned (16-byte aligned rows take the vector path).
 *   rows        0 returns at once; <= 2^31 - 1.
 *   vocab, d    as for rowstats_packed_embed_bytes.
 *   dtype       ROWSTATS_PROBS_BF16 or ROWSTATS_PROBS_FP16: of probs and of
 *               the packed table.
 *   packed      the table packed by rowstats_pack_embed with the same vocab
 *               and d.
 *   out         fp32 [rows, d] row-major, 16-byte aligned:
 *               out[r, j] = sum_c probs[r, c] * E[c, j], products exact in
 *               fp32, summed in fp32 in a fixed order (repeat calls give the
 *               same bits).
 *   Scratch: the library's grow-only buffer of partial products (8 [rows, d]
 *   fp32 tiles), shared with rowstats_selfcond and ordered with the other
 *   calls as described at the top. Errors: ROWSTATS_ERR_SHAPE, _DTYPE,
 *   _NULL, _HIP.
 */
int64_t rowstats_packed_embed_bytes(int64_t vocab, int64_t d);
int rowstats_pack_embed(const void *embed, int64_t vocab, int64_t d, int dtype,
                        void *packed, void *stream);
int rowstats_selfcond_product(const void *probs, int64_t probs_stride,
                              int64_t rows, int64_t vocab, int dtype,
                              const void *packed, int64_t d, float *out,
                              void *stream);

/*
 * Top-K logprobs of the rows of kept slots.
 * Defined by: diffusion_gemma_sampler page, stash_converged_logprobs
 * docstring (only the rows of converged slots are read, each scaled by
 * 1 / temperature; the K largest values, equal ones by lower id) and
 * the _lp_topk_kernel docstring (keys order by value, then by lower index,
 * so the top-K is unique; the K-th largest block maximum bounds it).
 *
 *   logits, row_stride, rows, vocab, temps, canvas_len  as for rowstats_run;
 *               T <= 0 is clamped to 1e-10 like the entropy's temperature.
 *   keep_mask   uint8 [ceil(rows / canvas_len)]: nonzero = slot kept.
 *   K           1 <= K <= vocab. K <= 64 runs the one-pass kernel (every row
 *               read once); larger K runs a separate kernel, one workgroup per
 *               kept row, that reads the row 4 times per 4096 keys.
 *   out_vals    fp32 [rows, K] row-major: out_vals[r, k] = s - log Z at the
 *               column of rank k (descending value, ties to lower column),
 *               log Z = log sum_c exp(s_c).
 *   out_idx     int64 [rows, K]: that column.
 *   Rows of slots that are not kept are not written.
 */
int topk_logprobs(const float *logits, int64_t row_stride, int64_t rows,
                  int64_t vocab, const float *temps, int64_t canvas_len,
                  const uint8_t *keep_mask, int32_t K, float *out_vals,
                  int64_t *out_idx, void *stream);

/*
 * The converged-logprob stash: for the rows of the kept requests, one stash
 * row each of the argmax, then the request's token ids or the num_topk
 * largest, then padding.
 * Defined by: diffusion_gemma_sampler page, stash_converged_logprobs
 * (docstring: for a kept request j, position p below valid[j] reads row
 * src[j] * canvas_len + p, scaled by 1 / temps[j], and writes
 * out_*[slots[j], p]; column 0 is the argmax, the next columns the
 * request's listed token ids or else its num_topk largest, equal values by
 * lower id, and the cells left token 0 at -inf; other requests are not
 * touched; launcher: num_topk + 1 <= width) and the
 * _lp_topk_kernel docstring (the key order). Where the page shows no body
 * this library reads it as stated below.
 *
 *   logits, row_stride, vocab  as for rowstats_run; logits_rows = rows of
 *               the matrix (>= 1).
 *   canvas_len  positions per request, >= 1; m * canvas_len <= 2^31 - 1.
 *   m           requests; m == 0 returns at once.
 *   src, slots, valid  int32 [m]. Request j with keep[j] != 0 owns the rows
 *               src[j] * canvas_len + p for 0 <= p < min(valid[j], canvas_len)
 *               (valid[j] <= 0: none); they go to stash slot slots[j],
 *               position p. A kept request with a row outside
 *               [0, logits_rows) or a slot outside [0, stash_slots) is
 *               skipped and flagged (rowstats_check_device).
 *   keep        uint8 [m]: nonzero = converged, written.
 *   temps       fp32 [m]: s = x / max(temps[j], 1e-10f) (IEEE fp32 division;
 *               T <= 0 uses 1e-10 as in rowstats_run's entropy).
 *   num_topk    0 <= num_topk <= vocab. Up to 64 the stash runs on the
 *               one-pass top-K kernel; above 64 on the workgroup-per-row
 *               kernel of topk_logprobs (the row read 4 times per 4096
 *               keys).
 *   num_token_ids, token_ids, token_ids_stride  NULL token_ids: no request
 *               has ids. Otherwise int32 num_token_ids [m] and token_ids
 *               [m, token_ids_stride] (row j at token_ids + j * stride):
 *               request j lists min(num_token_ids[j], stash_width - 1,
 *               token_ids_stride) ids when num_token_ids[j] > 0, else its
 *               num_topk largest. An id outside [0, vocab) is written as given
 *               with value -inf and flagged.
 *   stash_slots, stash_positions, stash_width  stash shape:
 *               stash_positions >= canvas_len, stash_width >= num_topk + 1.
 *   out_ids     int32 [stash_slots, stash_positions, stash_width] contiguous.
 *               Column 0: the argmax (lowest column attaining max s); then
 *               the ids, or the num_topk largest in descending key order
 *               (value, then lower column); the rest 0.
 *   out_logprobs fp32, same shape: s - log Z at each listed column (log Z =
 *               log sum_c exp(s_c)); with logits_mode != 0 the scaled logit s
 *               itself; -inf on padding.
 *   out_ranks   int32 [stash_slots, stash_positions]: the number of columns
 *               whose s is at least the argmax's (1 unless the maximum ties).
 *   Cells of requests not kept, and positions at or past valid[j], are not
 *   written.
 */
int stash_converged_logprobs(const float *logits, int64_t row_stride,
                             int64_t logits_rows, int64_t vocab,
                             int64_t canvas_len, int64_t m, const int32_t *src,
                             const int32_t *slots, const uint8_t *keep,
                             const int32_t *valid, const float *temps,
                             int32_t num_topk, const int32_t *num_token_ids,
                             const int32_t *token_ids, int64_t token_ids_stride,
                             int64_t stash_slots, int64_t stash_positions,
                             int32_t stash_width, int32_t *out_ids,
                             float *out_logprobs, int32_t *out_ranks,
                             int logits_mode, void *stream);

/* Text of the calling thread's last failure ("" if none). */
const char *rowstats_last_error(void);

/*
 * Synchronises `stream` and reports ROWSTATS_ERR_DEVICE if any kernel of
 * this library flagged a failure on the current device since the last
 * check: a bounded inter-workgroup wait that ran out (the outputs of that
 * call are then undefined), or a stash request or token id out of range
 * (that request or id was skipped, the rest is written). Clears the flag.
 */
int rowstats_check_device(void *stream);

/* Frees the library's scratch memory on every device (it is re-allocated on
 * the next call). Call only when no work of this library is in flight. */
int rowstats_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ROWSTATS_H */
