// C ABI of librowstats: argument checks, launch planning, per-device scratch
// and launches on the caller's stream. Declarations and contracts:
// include/rowstats.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "../../include/rowstats.h"
#include "rowstats_internal.h"
#include "topk_internal.h"

using namespace rowstats;

namespace {

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
// Start of the scratch buffer, for both entry points: the two row-claim
// counters (at the same place for every call, since each call zeroes the
// counter of the next one); the groups' row rings follow.
constexpr size_t kScratchHead = 256;
// Columns (and the padding columns of a row's last slice) index as int32 and
// the top-K key stores 0x7FFFFFFF - column: keep them all below 2^31.
constexpr int64_t kMaxVocab = 0x7FFFFFFFLL - 65536;

// Scratch of one device, grow-only, shared by both entry points: the
// waves' tagged summaries (row-statistics tuples or top-K records), row
// results and, for top-K, the kept-row list. Zeroed when allocated, after
// which tagged words are only ever told apart by the call epoch in their
// high half (epoch 0 never occurs; every call takes the next epoch).
struct DeviceState {
  bool ready = false;
  int cus = 0;
  int resident[2][3] = {};  // row-stats blocks per CU by [vector path][probs dtype]
  int topk_resident[2] = {};
  void *row_scratch = nullptr;
  size_t row_scratch_bytes = 0;
  uint32_t epoch = 0;       // epoch of the last call
  uint32_t *err_flag = nullptr;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

__global__ void fill_zero_u32(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t zero_async(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_u32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

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
    e = hipMalloc(&d.err_flag, sizeof(uint32_t));
    if (e != hipSuccess) return fail_hip(e, "hipMalloc(error flag)");
    e = hipMemset(d.err_flag, 0, sizeof(uint32_t));
    if (e != hipSuccess) return fail_hip(e, "hipMemset(error flag)");
    d.ready = true;
  }
  *out = &d;
  return ROWSTATS_OK;
}

int ensure_row_scratch(DeviceState &d, size_t bytes, hipStream_t s) {
  if (bytes <= d.row_scratch_bytes) return ROWSTATS_OK;
  hipError_t e;
  if (d.row_scratch) {
    e = hipFree(d.row_scratch);
    if (e != hipSuccess) return fail_hip(e, "hipFree(row scratch)");
    d.row_scratch = nullptr;
    d.row_scratch_bytes = 0;
  }
  size_t cap = bytes + bytes / 4;
  cap = (cap + 255) & ~(size_t)255;
  e = hipMalloc(&d.row_scratch, cap);
  if (e != hipSuccess) return fail_hip(e, "hipMalloc(row scratch)");
  d.row_scratch_bytes = cap;
  e = zero_async(reinterpret_cast<uint32_t *>(d.row_scratch), cap / 4, s);
  if (e != hipSuccess) return fail_hip(e, "zeroing row scratch");
  return ROWSTATS_OK;
}

// The epoch of a new call (clearing the scratch when the counter wraps).
int next_epoch(DeviceState &d, hipStream_t s, uint32_t *epoch) {
  if (++d.epoch == 0) {
    // the epoch wrapped: clear every tag it could still match
    hipError_t e = zero_async(reinterpret_cast<uint32_t *>(d.row_scratch), d.row_scratch_bytes / 4, s);
    if (e != hipSuccess) return fail_hip(e, "zeroing scratch");
    d.epoch = 1;
  }
  *epoch = d.epoch;
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

}  // namespace

extern "C" {

const char *rowstats_last_error(void) { return g_last_error.c_str(); }

int rowstats_run(const float *logits, int64_t row_stride, int64_t rows, int64_t vocab,
                 const float *temps, int64_t canvas_len, uint64_t seed, int probs_dtype,
                 int64_t *argmax, int64_t *sample, float *entropy, void *probs, void *stream) {
  g_last_error.clear();
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

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState *d = nullptr;
  if ((rc = device_state(&d))) return rc;

  RowStatsParams p = {};
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
  const int64_t waves = (int64_t)d->resident[p.vec_ok][probs_dtype] * d->cus * kWavesPerBlock;
  if (waves < 1) return fail(ROWSTATS_ERR_HIP, "row-stats kernel cannot be resident");
  if (p.C > waves)
    return fail(ROWSTATS_ERR_COOP,
                "vocab %lld needs %d co-resident waves per row, the device holds %lld",
                (long long)vocab, p.C, (long long)waves);
  int64_t groups = waves / p.C;
  if (groups > rows) groups = rows;
  p.n_groups = (int32_t)groups;
  const int64_t grid = (groups * p.C + kWavesPerBlock - 1) / kWavesPerBlock;

  const size_t head_bytes = kScratchHead + (size_t)groups * kRingBytes;
  const size_t tuple_bytes = (size_t)rows * p.C * kTupleBytes;
  const size_t rowres_bytes = (size_t)rows * kRowResultBytes;
  if ((rc = ensure_row_scratch(*d, head_bytes + tuple_bytes + rowres_bytes, s))) return rc;
  if ((rc = next_epoch(*d, s, &p.epoch))) return rc;
  char *base = reinterpret_cast<char *>(d->row_scratch);
  p.counters = reinterpret_cast<uint32_t *>(base);
  p.rings = reinterpret_cast<uint64_t *>(base + kScratchHead);
  p.tuples = reinterpret_cast<uint64_t *>(base + head_bytes);
  p.rowres = reinterpret_cast<uint64_t *>(base + head_bytes + tuple_bytes);
  p.err_flag = d->err_flag;
  hipError_t e = rowstats_launch(p, probs_dtype, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "row-stats kernel launch");
  return ROWSTATS_OK;
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
  if (K > kTopKMax) return fail(ROWSTATS_ERR_K, "K must be <= %d, got %d", kTopKMax, K);
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

  // As for rowstats_run: every wave resident, a row's C member waves at once.
  constexpr int kWavesPerBlock = kRowThreads / 64;
  const int64_t waves = (int64_t)d->topk_resident[p.vec_ok] * d->cus * kWavesPerBlock;
  if (waves < 1) return fail(ROWSTATS_ERR_HIP, "top-K kernel cannot be resident");
  if (p.C > waves || p.C > 64 * 64)
    return fail(ROWSTATS_ERR_COOP,
                "vocab %lld needs %d co-resident waves per row, the device holds %lld",
                (long long)vocab, p.C, (long long)waves);
  int64_t groups = waves / p.C;
  if (groups > rows) groups = rows;
  p.n_groups = (int32_t)groups;
  const int64_t grid = (groups * p.C + kWavesPerBlock - 1) / kWavesPerBlock;

  // records and row results are indexed by kept position (at most rows)
  const size_t head_bytes = kScratchHead + (size_t)groups * kRingBytes;
  const size_t record_bytes = (size_t)rows * p.C * topk_record_bytes(K);
  const size_t rowres_bytes = (size_t)rows * kRowResultBytes;
  const size_t kept_bytes = ((size_t)rows + 1) * sizeof(int64_t);
  const size_t temp_bytes = ((size_t)rows * sizeof(float) + 15) & ~(size_t)15;
  if ((rc = ensure_row_scratch(*d, head_bytes + record_bytes + rowres_bytes + kept_bytes + temp_bytes, s)))
    return rc;
  if ((rc = next_epoch(*d, s, &p.epoch))) return rc;
  char *base = reinterpret_cast<char *>(d->row_scratch);
  p.counters = reinterpret_cast<uint32_t *>(base);
  p.rings = reinterpret_cast<uint64_t *>(base + kScratchHead);
  base += head_bytes;
  p.records = reinterpret_cast<uint64_t *>(base);
  p.rowres = reinterpret_cast<uint64_t *>(base + record_bytes);
  p.kept_temp = reinterpret_cast<float *>(base + record_bytes + rowres_bytes);
  p.kept = reinterpret_cast<int64_t *>(base + record_bytes + rowres_bytes + temp_bytes);
  p.err_flag = d->err_flag;
  hipError_t e = topk_launch(p, (int)grid, s);
  if (e != hipSuccess) return fail_hip(e, "top-K kernel launch");
  return ROWSTATS_OK;
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
  e = hipMemcpy(&flag, d->err_flag, sizeof flag, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpy(error flag)");
  if (flag == 0) return ROWSTATS_OK;
  e = hipMemset(d->err_flag, 0, sizeof(uint32_t));
  if (e != hipSuccess) return fail_hip(e, "hipMemset(error flag)");
  return fail(ROWSTATS_ERR_DEVICE, "a kernel flagged an inter-workgroup wait that ran out (flag %u)",
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
    if (!d.ready) continue;
    if ((e = hipSetDevice(dev)) != hipSuccess) return fail_hip(e, "hipSetDevice");
    if (d.row_scratch) (void)hipFree(d.row_scratch);
    if (d.err_flag) (void)hipFree(d.err_flag);
    d = DeviceState();
  }
  if ((e = hipSetDevice(cur)) != hipSuccess) return fail_hip(e, "hipSetDevice");
  return ROWSTATS_OK;
}

}  // extern "C"
