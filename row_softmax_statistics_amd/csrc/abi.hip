// C ABI of librowstats: argument checks, launch planning, per-device scratch
// and launches on the caller's stream. Declarations and contracts:
// include/rowstats.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "../../include/rowstats.h"
#include "product_internal.h"
#include "rowstats_internal.h"
#include "selfcond_internal.h"
#include "topk_internal.h"

using namespace rowstats;

namespace {

// Scratch of rowstats_run_noalloc, one copy per GPU the library runs on,
// held until the process ends: zero when the code object is loaded, then
// only ever told apart by the epoch tags of its words (as the grow-only
// scratch below). Host code reaches it only through the address
// hipGetSymbolAddress gives for the current device.
constexpr size_t kNoAllocScratchBytes = ROWSTATS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint64_t scratch[kNoAllocScratchBytes / 8];

// Error words {report bits, epoch of the last call whose wait gave up} of
// the grow-only scratch [0] and of the fixed array above [1].
static __device__ __align__(16) uint32_t err_words[2][2];

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int fail_hip(hipError_t e, const char *what) {
  return fail(ROWSTATS_ERR_HIP, "%s: %s (hipError %d)", what, hipGetErrorString(e), (int)e);
}

constexpr int kMaxDevices = 64;
// Start of each scratch area, for both entry points: the two row-claim
// counters (at the same place for every call, since each call zeroes the
// counter of the next one); the groups' row rings follow.
constexpr size_t kScratchHead = 256;
// Columns (and the padding columns of a row's last slice) index as int32 and
// the top-K key stores 0x7FFFFFFF - column: keep them all below 2^31.
constexpr int64_t kMaxVocab = 0x7FFFFFFFLL - 65536;

// A scratch area: the waves' tagged summaries (row-statistics tuples or
// top-K records), row results and, for top-K, the kept-row list. Zero when
// it comes into use, after which tagged words are only ever told apart by
// the call epoch in their high half (epoch 0 never occurs; every call takes
// the next epoch, committed once its launch is queued).
struct Area {
  void *base = nullptr;
  size_t bytes = 0;
  uint32_t epoch = 0;        // epoch of the last queued call
  uint32_t *err = nullptr;   // its error words (device)
};

struct DeviceState {
  bool ready = false;
  int cus = 0;
  int resident[2][3] = {};  // row-stats blocks per CU by [vector path][probs dtype]
  int topk_resident[2] = {};
  Area grow;                // grow-only, shared by rowstats_run, topk_logprobs and the stash
  Area fixed;               // the fixed array of rowstats_run_noalloc
  // grow-only fp32 partial products of the two self-conditioning entry
  // points (untagged data, kept apart from the tagged words of `grow`)
  Area part;
  // The stream of the last call on the grow-only scratch; a call on another
  // stream first waits (on the device) for the work queued there so far.
  hipStream_t last_stream = nullptr;
  bool has_last = false;
  hipEvent_t order_event = nullptr;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

__global__ void fill_zero_u32(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Zeroes n words with a fill kernel (no memset node, so it also records
// correctly into a captured graph).
hipError_t zero_async(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_u32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

// Per-device set-up, once per device with it current: occupancy of every
// kernel variant and the device addresses of the fixed scratch array and
// the error words. Allocates nothing.
int device_state(DeviceState **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ROWSTATS_ERR_HIP, "device %d out of range", dev);
  DeviceState &d = g_dev[dev];
  if (!d.ready) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    d.cus = prop.multiProcessorCount;
    for (int vec = 0; vec < 2; ++vec) {
      for (int k = 0; k < 3; ++k) {
        e = rowstats_resident_blocks(k, vec != 0, &d.resident[vec][k]);
        if (e != hipSuccess) return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
      }
      e = topk_resident_blocks(vec != 0, &d.topk_resident[vec]);
      if (e != hipSuccess) return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    }
    void *fixed = nullptr, *err = nullptr;
    e = hipGetSymbolAddress(&fixed, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    e = hipGetSymbolAddress(&err, HIP_SYMBOL(err_words));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(error words)");
    d.fixed.base = fixed;
    d.fixed.bytes = kNoAllocScratchBytes;
    d.grow.err = static_cast<uint32_t *>(err);
    d.fixed.err = static_cast<uint32_t *>(err) + 2;
    d.ready = true;
  }
  *out = &d;
  return ROWSTATS_OK;
}

int ensure_grow_scratch(DeviceState &d, size_t bytes, hipStream_t s) {
  Area &a = d.grow;
  if (bytes <= a.bytes) return ROWSTATS_OK;
  hipError_t e;
  if (a.base) {
    e = hipFree(a.base);  // waits for the work that may still use it
    if (e != hipSuccess) return fail_hip(e, "hipFree(row scratch)");
    a.base = nullptr;
    a.bytes = 0;
  }
  size_t cap = bytes + bytes / 4;
  cap = (cap + 255) & ~(size_t)255;
  e = hipMalloc(&a.base, cap);
  if (e != hipSuccess) return fail_hip(e, "hipMalloc(row scratch)");
  a.bytes = cap;
  e = zero_async(reinterpret_cast<uint32_t *>(a.base), cap / 4, s);
  if (e != hipSuccess) return fail_hip(e, "zeroing row scratch");
  return ROWSTATS_OK;
}

// The epoch of a new call on area a. When the counter wraps, the area and
// its failed-epoch word are cleared first, since old tags could match again.
int next_epoch(Area &a, hipStream_t s, uint32_t *epoch) {
  uint32_t e = a.epoch + 1;
  if (e == 0) {
    hipError_t h = zero_async(reinterpret_cast<uint32_t *>(a.base), a.bytes / 4, s);
    if (h == hipSuccess) h = zero_async(a.err + 1, 1, s);
    if (h != hipSuccess) return fail_hip(h, "zeroing scratch");
    e = 1;
  }
  *epoch = e;
  return ROWSTATS_OK;
}

// Grow-only buffer of the self-conditioning partial products (no zeroing:
// every element a call reads it has written first).
int ensure_partials(DeviceState &d, size_t bytes) {
  Area &a = d.part;
  if (bytes <= a.bytes) return ROWSTATS_OK;
  hipError_t e;
  if (a.base) {
    e = hipFree(a.base);  // waits for the work that may still use it
    if (e != hipSuccess) return fail_hip(e, "hipFree(partial products)");
    a.base = nullptr;
    a.bytes = 0;
  }
  size_t cap = bytes + bytes / 4;
  cap = (cap + 255) & ~(size_t)255;
  e = hipMalloc(&a.base, cap);
  if (e != hipSuccess) return fail_hip(e, "hipMalloc(partial products)");
  a.bytes = cap;
  return ROWSTATS_OK;
}

// Orders a call on the grow-only scratch after the last call queued on
// another stream (they share the scratch and its row-claim counters): the
// event recorded after every launch on the grow-only scratch.
int order_after_last(DeviceState &d, hipStream_t s) {
  if (d.has_last && d.last_stream != s) {
    hipError_t e = hipStreamWaitEvent(s, d.order_event, 0);
    if (e != hipSuccess) return fail_hip(e, "waiting for the previous call's stream");
  }
  return ROWSTATS_OK;
}

int note_stream(DeviceState &d, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (!d.order_event) e = hipEventCreateWithFlags(&d.order_event, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(d.order_event, s);
  if (e != hipSuccess) {
    d.has_last = false;
    return fail_hip(e, "recording the call's completion event");
  }
  d.last_stream = s;
  d.has_last = true;
  return ROWSTATS_OK;
}

int check_common(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                 const float *temps, int64_t canvas_len) {
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(ROWSTATS_ERR_SHAPE, "vocab must be in [1, %lld], got %lld", (long long)kMaxVocab,
                (long long)vocab);
  if (row_stride < vocab)
    return fail(ROWSTATS_ERR_SHAPE, "row_stride %lld < vocab %lld", (long long)row_stride,
                (long long)vocab);
  if (canvas_len < 1)
    return fail(ROWSTATS_ERR_SHAPE, "canvas_len must be >= 1, got %lld", (long long)canvas_len);
  if (!logits) return fail(ROWSTATS_ERR_NULL, "logits is NULL");
  if (!temps) return fail(ROWSTATS_ERR_NULL, "temps is NULL");
  // rows are handed out as 32-bit positions
  if (rows > 0x7FFFFFFFLL)
    return fail(ROWSTATS_ERR_SHAPE, "rows must be <= 2^31 - 1, got %lld", (long long)rows);
  return ROWSTATS_OK;
}

// Groups, scratch layout and launch of the top-K kernel (both entry
// points); p.rows is the most rows the call can keep.
int plan_and_launch_topk(DeviceState &d, TopKParams &p, hipStream_t s) {
  // As for rowstats_run: every wave resident, a row's C member waves at once.
  constexpr int kWavesPerBlock = kRowThreads / 64;
  const int64_t rows = p.rows;
  const int64_t waves = (int64_t)d.topk_resident[p.vec_ok] * d.cus * kWavesPerBlock;
  if (waves < 1) return fail(ROWSTATS_ERR_HIP, "top-K kernel cannot be resident");
  if (p.C > waves || p.C > 64 * 64)
    return fail(ROWSTATS_ERR_COOP,
                "vocab %d needs %d co-resident waves per row, the device holds %lld", p.vocab,
                p.C, (long long)waves);
  int64_t groups = waves / p.C;
  if (groups > rows) groups = rows;
  p.n_groups = (int32_t)groups;
  const int64_t grid = (groups * p.C + kWavesPerBlock - 1) / kWavesPerBlock;

  // records and row results are indexed by kept position (at most rows)
  auto align16 = [](size_t b) { return (b + 15) & ~(size_t)15; };
  const size_t head_bytes = kScratchHead + (size_t)groups * kRingBytes;
  const size_t record_bytes = (size_t)rows * p.C * topk_record_bytes(p.K);
  const size_t rowres_bytes = (size_t)rows * kRowResultBytes;
  const size_t temp_bytes = align16((size_t)rows * sizeof(float));
  const size_t kept_bytes = align16(((size_t)rows + 1) * sizeof(int64_t));
  const size_t dst_bytes = p.stash ? (size_t)rows * sizeof(int64_t) : 0;
  const size_t req_bytes = p.stash ? align16((size_t)rows * sizeof(int32_t)) : 0;
  int rc = order_after_last(d, s);
  if (rc) return rc;
  rc = ensure_grow_scratch(d, head_bytes + record_bytes + rowres_bytes + temp_bytes +
                                  kept_bytes + dst_bytes + req_bytes, s);
  if (rc) return rc;
  if ((rc = next_epoch(d.grow, s, &p.epoch))) return rc;
  char *base = reinterpret_cast<char *>(d.grow.base);
  p.counters = reinterpret_cast<uint32_t *>(base);
  p.rings = reinterpret_cast<uint64_t *>(base + kScratchHead);
  base += head_bytes;
  p.records = reinterpret_cast<uint64_t *>(base);
  base += record_bytes;
  p.rowres = reinterpret_cast<uint64_t *>(base);
  base += rowres_bytes;
  p.kept_temp = reinterpret_cast<float *>(base);
  base += temp_bytes;
  p.kept = reinterpret_cast<int64_t *>(base);
  base += kept_bytes;
  p.kept_dst = p.stash ? reinterpret_cast<int64_t *>(base) : nullptr;
  base += dst_bytes;
  p.kept_req = p.stash ? reinterpret_cast<int32_t *>(base) : nullptr;
  p.err_flag = d.grow.err;
  hipError_t e = topk_launch(p, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "top-K kernel launch");
  d.grow.epoch = p.epoch;
  return note_stream(d, s);
}

// Scratch layout and launches of the top-K path for K > kTopKMax (and the
// stash for num_topk > kTopKMax): the kept-row list, temperatures and, for
// the stash, stash rows and requests after the scratch head (whose
// row-claim counters the pre-pass zeroes, as for every top-K call).
int plan_and_launch_topk_wide(DeviceState &d, TopKParams &p, hipStream_t s) {
  auto align16 = [](size_t b) { return (b + 15) & ~(size_t)15; };
  const size_t temp_bytes = align16((size_t)p.rows * sizeof(float));
  const size_t kept_bytes = align16(((size_t)p.rows + 1) * sizeof(int64_t));
  const size_t dst_bytes = p.stash ? (size_t)p.rows * sizeof(int64_t) : 0;
  const size_t req_bytes = p.stash ? align16((size_t)p.rows * sizeof(int32_t)) : 0;
  int rc = order_after_last(d, s);
  if (rc) return rc;
  if ((rc = ensure_grow_scratch(d, kScratchHead + temp_bytes + kept_bytes + dst_bytes + req_bytes,
                                s)))
    return rc;
  char *base = reinterpret_cast<char *>(d.grow.base);
  p.counters = reinterpret_cast<uint32_t *>(base);
  base += kScratchHead;
  p.kept_temp = reinterpret_cast<float *>(base);
  base += temp_bytes;
  p.kept = reinterpret_cast<int64_t *>(base);
  base += kept_bytes;
  p.kept_dst = p.stash ? reinterpret_cast<int64_t *>(base) : nullptr;
  base += dst_bytes;
  p.kept_req = p.stash ? reinterpret_cast<int32_t *>(base) : nullptr;
  p.err_flag = d.grow.err;
  hipError_t e = topk_wide_launch(p, s);
  if (e != hipSuccess) return fail_hip(e, "top-K kernel launch");
  return note_stream(d, s);
}

// Checks and launch plan of a row-statistics call, shared by rowstats_run
// and rowstats_run_noalloc: fills p except the scratch pointers and the
// epoch, and returns the grid and the scratch bytes the call needs.
int plan_rowstats(const DeviceState &d, const float *logits, int64_t row_stride, int64_t rows,
                  int64_t vocab, const float *temps, int64_t canvas_len, uint64_t seed,
                  int probs_dtype, int64_t *argmax, int64_t *sample, float *entropy, void *probs,
                  RowStatsParams &p, int64_t *grid, size_t *need, size_t *head_bytes,
                  size_t *tuple_bytes) {
  p = RowStatsParams{};
  p.logits = logits;
  p.ld = row_stride;
  p.rows = rows;
  p.vocab = (int32_t)vocab;
  p.C = (int32_t)((vocab + kChunkCols - 1) / kChunkCols);
  p.vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) && (row_stride % 4 == 0) &&
             (vocab % 4 == 0) && ((reinterpret_cast<uintptr_t>(probs) & 7) == 0);
  p.temps = temps;
  p.canvas_len = canvas_len;
  slot_divider(canvas_len, &p.slot_mul, &p.slot_shift);
  p.seed = seed;
  p.argmax = argmax;
  p.sample = sample;
  p.entropy = entropy;
  p.probs = probs;

  // Every wave of the launch is resident (cooperative launch); the C waves
  // of a row's group keep their chunks in registers until the row is
  // merged, so a group must fit.
  constexpr int kWavesPerBlock = kRowThreads / 64;
  const int64_t waves = (int64_t)d.resident[p.vec_ok][probs_dtype] * d.cus * kWavesPerBlock;
  if (waves < 1) return fail(ROWSTATS_ERR_HIP, "row-stats kernel cannot be resident");
  if (p.C > waves)
    return fail(ROWSTATS_ERR_COOP,
                "vocab %lld needs %d co-resident waves per row, the device holds %lld",
                (long long)vocab, p.C, (long long)waves);
  int64_t groups = waves / p.C;
  if (groups > rows) groups = rows;
  p.n_groups = (int32_t)groups;
  *grid = (groups * p.C + kWavesPerBlock - 1) / kWavesPerBlock;
  *head_bytes = kScratchHead + (size_t)groups * kRingBytes;
  *tuple_bytes = (size_t)rows * p.C * kTupleBytes;
  *need = *head_bytes + *tuple_bytes + (size_t)rows * kRowResultBytes;
  return ROWSTATS_OK;
}

// Argument checks of rowstats_run that need no device.
int check_rowstats_args(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                        const float *temps, int64_t canvas_len, int probs_dtype,
                        const int64_t *argmax, const int64_t *sample, const float *entropy,
                        const void *probs) {
  if (probs_dtype < ROWSTATS_PROBS_NONE || probs_dtype > ROWSTATS_PROBS_FP16)
    return fail(ROWSTATS_ERR_DTYPE, "probs_dtype must be 0 (none), 1 (bf16) or 2 (fp16), got %d",
                probs_dtype);
  if (rows < 0) return fail(ROWSTATS_ERR_SHAPE, "rows must be >= 0, got %lld", (long long)rows);
  if (rows == 0) return ROWSTATS_OK;
  int rc = check_common(logits, row_stride, rows, vocab, temps, canvas_len);
  if (rc) return rc;
  if (!argmax || !sample || !entropy) return fail(ROWSTATS_ERR_NULL, "an output pointer is NULL");
  if (probs_dtype != ROWSTATS_PROBS_NONE && !probs)
    return fail(ROWSTATS_ERR_NULL, "probs is NULL but probs_dtype asks for probabilities");
  return ROWSTATS_OK;
}

void set_scratch(RowStatsParams &p, const Area &a, size_t head_bytes, size_t tuple_bytes) {
  char *base = reinterpret_cast<char *>(a.base);
  p.counters = reinterpret_cast<uint32_t *>(base);
  p.rings = reinterpret_cast<uint64_t *>(base + kScratchHead);
  p.tuples = reinterpret_cast<uint64_t *>(base + head_bytes);
  p.rowres = reinterpret_cast<uint64_t *>(base + head_bytes + tuple_bytes);
  p.err_flag = a.err;
}

}  // namespace

extern "C" {

const char *rowstats_last_error(void) { return g_last_error.c_str(); }

int rowstats_run(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                 const float *temps, int64_t canvas_len, uint64_t seed, int probs_dtype,
                 int64_t *argmax, int64_t *sample, float *entropy, void *probs, void *stream) {
  g_last_error.clear();
  int rc = check_rowstats_args(logits, row_stride, rows, vocab, temps, canvas_len, probs_dtype,
                               argmax, sample, entropy, probs);
  if (rc || rows == 0) return rc;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  if ((rc = device_state(&d))) return rc;
  RowStatsParams p;
  int64_t grid = 0;
  size_t need = 0, head_bytes = 0, tuple_bytes = 0;
  if ((rc = plan_rowstats(*d, logits, row_stride, rows, vocab, temps, canvas_len, seed, probs_dtype,
                          argmax, sample, entropy, probs, p, &grid, &need, &head_bytes,
                          &tuple_bytes)))
    return rc;
  if ((rc = order_after_last(*d, s))) return rc;
  if ((rc = ensure_grow_scratch(*d, need, s))) return rc;
  if ((rc = next_epoch(d->grow, s, &p.epoch))) return rc;
  set_scratch(p, d->grow, head_bytes, tuple_bytes);
  hipError_t e = rowstats_launch(p, probs_dtype, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "row-stats kernel launch");
  d->grow.epoch = p.epoch;
  return note_stream(*d, s);
}

int rowstats_run_noalloc(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                         const float *temps, int64_t canvas_len, uint64_t seed, int probs_dtype,
                         int64_t *argmax, int64_t *sample, float *entropy, void *probs,
                         void *stream) {
  g_last_error.clear();
  int rc = check_rowstats_args(logits, row_stride, rows, vocab, temps, canvas_len, probs_dtype,
                               argmax, sample, entropy, probs);
  if (rc || rows == 0) return rc;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  if ((rc = device_state(&d))) return rc;
  RowStatsParams p;
  int64_t grid = 0;
  size_t need = 0, head_bytes = 0, tuple_bytes = 0;
  if ((rc = plan_rowstats(*d, logits, row_stride, rows, vocab, temps, canvas_len, seed, probs_dtype,
                          argmax, sample, entropy, probs, p, &grid, &need, &head_bytes,
                          &tuple_bytes)))
    return rc;
  if (need > d->fixed.bytes)
    return fail(ROWSTATS_ERR_SCRATCH,
                "%lld rows of %d chunks need %zu bytes of scratch; the fixed array holds %zu",
                (long long)rows, p.C, need, d->fixed.bytes);
  if ((rc = next_epoch(d->fixed, s, &p.epoch))) return rc;
  set_scratch(p, d->fixed, head_bytes, tuple_bytes);
  // The part of the array this call uses, and the failed-epoch word, start
  // at zero (fill kernels, no memset node): a captured call replays with the
  // epoch of its capture, and the clearing keeps the words of an earlier
  // replay from passing for this one's.
  hipError_t e = zero_async(reinterpret_cast<uint32_t *>(d->fixed.base), need / 4, s);
  if (e == hipSuccess) e = zero_async(d->fixed.err + 1, 1, s);
  if (e != hipSuccess) return fail_hip(e, "clearing the fixed scratch");
  e = rowstats_launch(p, probs_dtype, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "row-stats kernel launch");
  d->fixed.epoch = p.epoch;
  return ROWSTATS_OK;
}

int rowstats_selfcond(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                      const float *temps, int64_t canvas_len, uint64_t seed, int dtype,
                      const void *embed, int64_t d, int64_t *argmax, int64_t *sample,
                      float *entropy, float *out, void *stream) {
  g_last_error.clear();
  int rc = check_rowstats_args(logits, row_stride, rows, vocab, temps, canvas_len,
                               ROWSTATS_PROBS_NONE, argmax, sample, entropy, nullptr);
  if (rc || rows == 0) return rc;
  if (dtype != ROWSTATS_PROBS_BF16 && dtype != ROWSTATS_PROBS_FP16)
    return fail(ROWSTATS_ERR_DTYPE, "dtype must be ROWSTATS_PROBS_BF16 or _FP16, got %d", dtype);
  if (!embed || !out) return fail(ROWSTATS_ERR_NULL, "embed or out is NULL");
  if (d < kSelfCondDMultiple || d % kSelfCondDMultiple != 0 || d > (1 << 20))
    return fail(ROWSTATS_ERR_SHAPE, "d must be a multiple of %d in [%d, 2^20], got %lld",
                kSelfCondDMultiple, kSelfCondDMultiple, (long long)d);
  if ((reinterpret_cast<uintptr_t>(embed) & 15) || (reinterpret_cast<uintptr_t>(out) & 15))
    return fail(ROWSTATS_ERR_SHAPE, "embed and out must be 16-byte aligned");
  const int64_t m_tiles = (rows + kSelfCondTileM - 1) / kSelfCondTileM;
  const int64_t n_tiles = (d + kSelfCondTileN - 1) / kSelfCondTileN;
  if ((int64_t)kSelfCondSplits * m_tiles * n_tiles > 0x7FFFFFFFLL)
    return fail(ROWSTATS_ERR_SHAPE, "rows %lld x d %lld is too large", (long long)rows,
                (long long)d);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *dev = nullptr;
  if ((rc = device_state(&dev))) return rc;
  RowStatsParams p;
  int64_t grid = 0;
  size_t need = 0, head_bytes = 0, tuple_bytes = 0;
  if ((rc = plan_rowstats(*dev, logits, row_stride, rows, vocab, temps, canvas_len, seed,
                          ROWSTATS_PROBS_NONE, argmax, sample, entropy, nullptr, p, &grid, &need,
                          &head_bytes, &tuple_bytes)))
    return rc;
  const size_t partial_bytes = (size_t)kSelfCondSplits * rows * d * sizeof(float);
  if ((rc = order_after_last(*dev, s))) return rc;
  if ((rc = ensure_grow_scratch(*dev, need, s))) return rc;
  if ((rc = ensure_partials(*dev, partial_bytes))) return rc;
  if ((rc = next_epoch(dev->grow, s, &p.epoch))) return rc;
  set_scratch(p, dev->grow, head_bytes, tuple_bytes);
  hipError_t e = rowstats_launch(p, ROWSTATS_PROBS_NONE, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "row-stats kernel launch");

  SelfCondParams q = {};
  q.logits = logits;
  q.ld = row_stride;
  q.rows = rows;
  q.vocab = (int32_t)vocab;
  q.d = (int32_t)d;
  q.temps = temps;
  q.slot_mul = p.slot_mul;
  q.slot_shift = p.slot_shift;
  q.rowres = p.rowres;
  q.E = static_cast<const uint16_t *>(embed);
  q.partial = static_cast<float *>(dev->part.base);
  q.out = out;
  const int64_t per = (vocab + kSelfCondSplits - 1) / kSelfCondSplits;
  q.k_per_split = (int32_t)((per + kSelfCondStepK - 1) / kSelfCondStepK * kSelfCondStepK);
  q.m_tiles = (int32_t)m_tiles;
  q.n_tiles = (int32_t)n_tiles;
  q.vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) && (row_stride % 4 == 0);
  q.f16 = dtype == ROWSTATS_PROBS_FP16;
  e = selfcond_launch(q, s);
  if (e != hipSuccess) return fail_hip(e, "self-conditioning kernel launch");
  dev->grow.epoch = p.epoch;
  return note_stream(*dev, s);
}

int64_t rowstats_packed_embed_bytes(int64_t vocab, int64_t d) {
  g_last_error.clear();
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(ROWSTATS_ERR_SHAPE, "vocab must be in [1, %lld], got %lld", (long long)kMaxVocab,
                (long long)vocab);
  if (d < kProductDMultiple || d % kProductDMultiple != 0 || d > (1 << 20))
    return fail(ROWSTATS_ERR_SHAPE, "d must be a multiple of %d in [%d, 2^20], got %lld",
                kProductDMultiple, kProductDMultiple, (long long)d);
  return packed_embed_bytes(vocab, d);
}

int rowstats_pack_embed(const void *embed, int64_t vocab, int64_t d, int dtype, void *packed,
                        void *stream) {
  const int64_t bytes = rowstats_packed_embed_bytes(vocab, d);
  if (bytes < 0) return (int)bytes;
  if (dtype != ROWSTATS_PROBS_BF16 && dtype != ROWSTATS_PROBS_FP16)
    return fail(ROWSTATS_ERR_DTYPE, "dtype must be ROWSTATS_PROBS_BF16 or _FP16, got %d", dtype);
  if (!embed || !packed) return fail(ROWSTATS_ERR_NULL, "embed or packed is NULL");
  if ((reinterpret_cast<uintptr_t>(embed) & 1) || (reinterpret_cast<uintptr_t>(packed) & 15))
    return fail(ROWSTATS_ERR_SHAPE, "embed must be 2-byte and packed 16-byte aligned");
  hipError_t e = pack_embed_launch(static_cast<const uint16_t *>(embed), vocab, d,
                                   static_cast<uint16_t *>(packed),
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "packing kernel launch");
  return ROWSTATS_OK;
}

int rowstats_selfcond_product(const void *probs, int64_t probs_stride, int64_t rows,
                              int64_t vocab, int dtype, const void *packed, int64_t d,
                              float *out, void *stream) {
  g_last_error.clear();
  if (rows < 0 || rows > 0x7FFFFFFFLL)
    return fail(ROWSTATS_ERR_SHAPE, "rows must be in [0, 2^31 - 1], got %lld", (long long)rows);
  if (rows == 0) return ROWSTATS_OK;
  if (rowstats_packed_embed_bytes(vocab, d) < 0) return ROWSTATS_ERR_SHAPE;
  if (probs_stride < vocab)
    return fail(ROWSTATS_ERR_SHAPE, "probs_stride %lld < vocab %lld", (long long)probs_stride,
                (long long)vocab);
  if (dtype != ROWSTATS_PROBS_BF16 && dtype != ROWSTATS_PROBS_FP16)
    return fail(ROWSTATS_ERR_DTYPE, "dtype must be ROWSTATS_PROBS_BF16 or _FP16, got %d", dtype);
  if (!probs || !packed || !out) return fail(ROWSTATS_ERR_NULL, "probs, packed or out is NULL");
  if ((reinterpret_cast<uintptr_t>(probs) & 1) || (reinterpret_cast<uintptr_t>(packed) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return fail(ROWSTATS_ERR_SHAPE, "probs must be 2-byte, packed and out 16-byte aligned");
  const int64_t m_tiles = (rows + kProductTileM - 1) / kProductTileM;
  const int64_t n_tiles = (d + kProductTileN - 1) / kProductTileN;
  if ((int64_t)kProductSplits * m_tiles * n_tiles > 0x7FFFFFFFLL)
    return fail(ROWSTATS_ERR_SHAPE, "rows %lld x d %lld is too large", (long long)rows,
                (long long)d);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *dev = nullptr;
  int rc;
  if ((rc = device_state(&dev))) return rc;
  if ((rc = order_after_last(*dev, s))) return rc;
  if ((rc = ensure_partials(*dev, (size_t)kProductSplits * rows * d * sizeof(float)))) return rc;
  ProductParams q = {};
  q.P = static_cast<const uint16_t *>(probs);
  q.ldp = probs_stride;
  q.rows = rows;
  q.vocab = (int32_t)vocab;
  q.d = (int32_t)d;
  q.packed = static_cast<const uint16_t *>(packed);
  q.partial = static_cast<float *>(dev->part.base);
  q.out = out;
  const int64_t per = (vocab + kProductSplits - 1) / kProductSplits;
  q.k_per_split = (int32_t)((per + kProductStepK - 1) / kProductStepK * kProductStepK);
  q.m_tiles = (int32_t)m_tiles;
  q.n_tiles = (int32_t)n_tiles;
  q.vec_ok = ((reinterpret_cast<uintptr_t>(probs) & 15) == 0) && (probs_stride % 8 == 0);
  q.f16 = dtype == ROWSTATS_PROBS_FP16;
  hipError_t e = product_launch(q, s);
  if (e != hipSuccess) return fail_hip(e, "self-conditioning product launch");
  return note_stream(*dev, s);
}

int topk_logprobs(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                  const float *temps, int64_t canvas_len, const uint8_t *keep_mask, int32_t K,
                  float *out_vals, int64_t *out_idx, void *stream) {
  g_last_error.clear();
  if (rows < 0) return fail(ROWSTATS_ERR_SHAPE, "rows must be >= 0, got %lld", (long long)rows);
  if (rows == 0) return ROWSTATS_OK;
  int rc = check_common(logits, row_stride, rows, vocab, temps, canvas_len);
  if (rc) return rc;
  if (K < 1 || (int64_t)K > vocab)
    return fail(ROWSTATS_ERR_K, "K must be in [1, vocab=%lld], got %d", (long long)vocab, K);
  if (!keep_mask) return fail(ROWSTATS_ERR_NULL, "keep_mask is NULL");
  if (!out_vals || !out_idx) return fail(ROWSTATS_ERR_NULL, "an output pointer is NULL");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  if ((rc = device_state(&d))) return rc;

  TopKParams p = {};
  p.logits = logits;
  p.ld = row_stride;
  p.rows = rows;
  p.vocab = (int32_t)vocab;
  p.C = (int32_t)((vocab + kChunkCols - 1) / kChunkCols);
  p.vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) && (row_stride % 4 == 0) &&
             (vocab % 4 == 0);
  p.K = K;
  p.temps = temps;
  p.canvas_len = canvas_len;
  p.keep = keep_mask;
  p.out_vals = out_vals;
  p.out_idx = out_idx;

  if (K > kTopKMax) return plan_and_launch_topk_wide(*d, p, s);
  return plan_and_launch_topk(*d, p, s);
}

int stash_converged_logprobs(const float *logits, int64_t row_stride, int64_t logits_rows,
                             int64_t vocab, int64_t canvas_len, int64_t m, const int32_t *src,
                             const int32_t *slots, const uint8_t *keep, const int32_t *valid,
                             const float *temps, int32_t num_topk, const int32_t *num_token_ids,
                             const int32_t *token_ids, int64_t token_ids_stride,
                             int64_t stash_slots, int64_t stash_positions, int32_t stash_width,
                             int32_t *out_ids, float *out_logprobs, int32_t *out_ranks,
                             int logits_mode, void *stream) {
  g_last_error.clear();
  if (m < 0) return fail(ROWSTATS_ERR_SHAPE, "m must be >= 0, got %lld", (long long)m);
  if (m == 0) return ROWSTATS_OK;
  if (logits_rows < 1)
    return fail(ROWSTATS_ERR_SHAPE, "logits_rows must be >= 1, got %lld", (long long)logits_rows);
  int rc = check_common(logits, row_stride, logits_rows, vocab, temps, canvas_len);
  if (rc) return rc;
  if (canvas_len > 0x7FFFFFFFLL / m)
    return fail(ROWSTATS_ERR_SHAPE, "m * canvas_len must be <= 2^31 - 1, got %lld * %lld",
                (long long)m, (long long)canvas_len);
  if (num_topk < 0 || (int64_t)num_topk > vocab)
    return fail(ROWSTATS_ERR_K, "num_topk must be in [0, vocab=%lld], got %d", (long long)vocab,
                num_topk);
  if ((int64_t)stash_width < (int64_t)num_topk + 1)
    return fail(ROWSTATS_ERR_SHAPE, "stash_width %d < num_topk + 1 = %d", stash_width,
                num_topk + 1);
  if (stash_slots < 1)
    return fail(ROWSTATS_ERR_SHAPE, "stash_slots must be >= 1, got %lld", (long long)stash_slots);
  if (stash_positions < canvas_len)
    return fail(ROWSTATS_ERR_SHAPE, "stash_positions %lld < canvas_len %lld",
                (long long)stash_positions, (long long)canvas_len);
  if (!src || !slots || !keep || !valid)
    return fail(ROWSTATS_ERR_NULL, "src, slots, keep or valid is NULL");
  if (!out_ids || !out_logprobs || !out_ranks)
    return fail(ROWSTATS_ERR_NULL, "an output pointer is NULL");
  if (token_ids) {
    if (!num_token_ids) return fail(ROWSTATS_ERR_NULL, "token_ids given without num_token_ids");
    if (token_ids_stride < 1)
      return fail(ROWSTATS_ERR_SHAPE, "token_ids_stride must be >= 1, got %lld",
                  (long long)token_ids_stride);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  if ((rc = device_state(&d))) return rc;

  TopKParams p = {};
  p.logits = logits;
  p.ld = row_stride;
  p.rows = m * canvas_len;  // most rows the kept requests can own
  p.vocab = (int32_t)vocab;
  p.C = (int32_t)((vocab + kChunkCols - 1) / kChunkCols);
  p.vec_ok = ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) && (row_stride % 4 == 0) &&
             (vocab % 4 == 0);
  // two keys at least, so that the ties at the maximum are known without a
  // recount unless the two largest tie
  p.K = (int32_t)(vocab < 2 ? vocab : (num_topk < 2 ? 2 : num_topk));
  p.temps = temps;
  p.canvas_len = canvas_len;
  p.keep = keep;
  p.stash = 1;
  p.K_out = num_topk;
  p.logits_mode = logits_mode != 0;
  p.width = stash_width;
  p.m = m;
  p.logits_rows = logits_rows;
  p.stash_slots = stash_slots;
  p.positions = stash_positions;
  p.src = src;
  p.slots = slots;
  p.valid = valid;
  p.num_ids = token_ids ? num_token_ids : nullptr;
  p.ids = token_ids;
  p.ids_stride = token_ids ? token_ids_stride : 0;
  p.out_ids32 = out_ids;
  p.out_lp = out_logprobs;
  p.out_ranks = out_ranks;
  if (num_topk > kTopKMax) return plan_and_launch_topk_wide(*d, p, s);
  return plan_and_launch_topk(*d, p, s);
}

int rowstats_check_device(void *stream) {
  g_last_error.clear();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  int rc = device_state(&d);
  if (rc) return rc;
  uint32_t flag = 0;
  for (Area *a : {&d->grow, &d->fixed}) {
    uint32_t f = 0;
    e = hipMemcpy(&f, a->err, sizeof f, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpy(error flag)");
    if (f != 0) {
      e = hipMemset(a->err, 0, sizeof(uint32_t));
      if (e != hipSuccess) return fail_hip(e, "hipMemset(error flag)");
    }
    flag |= f;
  }
  if (flag == 0) return ROWSTATS_OK;
  return fail(ROWSTATS_ERR_DEVICE, "a kernel flagged %s (flag %u)",
              (flag & kErrWait) ? "an inter-workgroup wait that ran out"
                                : "a stash index out of range (request or token id skipped)",
              flag);
}

int rowstats_release(void) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    DeviceState &d = g_dev[dev];
    if (!d.ready || (!d.grow.base && !d.part.base && !d.order_event)) continue;
    if ((e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e, "hipSetDevice");
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
    if (d.grow.base) (void)hipFree(d.grow.base);
    if (d.part.base) (void)hipFree(d.part.base);
    if (d.order_event) (void)hipEventDestroy(d.order_event);
    // the next call on the grow-only scratch allocates it afresh (zeroed);
    // the epoch keeps counting
    d.grow.base = nullptr;
    d.grow.bytes = 0;
    d.part.base = nullptr;
    d.part.bytes = 0;
    d.order_event = nullptr;
    d.has_last = false;
  }
  if ((e = hipSetDevice(cur)) != hipSuccess) return fail_hip(e, "hipSetDevice");
  return ROWSTATS_OK;
}

}  // extern "C"
