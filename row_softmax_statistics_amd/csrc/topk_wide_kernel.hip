// Top-K logprobs for K above what the one-pass top-K kernel holds (K > 64,
// up to the vocabulary): one workgroup per kept row, exact, in passes over
// the row.
//
// Method: vLLM API page "diffusion_gemma_sampler", stash_converged_logprobs
// docstring (kept rows divided by their temperature; the K largest, ties to
// the lower id) and the _lp_topk_kernel docstring (keys ordered by value,
// then by lower index, so the top-K is unique).
//
// Per row (1024 threads, four consecutive columns per thread and tile), in
// batches of up to kBatch keys below the previous batch's smallest:
//   1. the value v of the batch's last key by a radix select over the
//      32-bit order-preserving value keys: digits of 11, 11 and 10 bits,
//      one pass over the row each with a histogram in LDS; the first batch's
//      first pass also forms the row maximum m and S = sum exp(s - m)
//      (online: each thread rescales its sum when its maximum rises);
//   2. one pass collecting the keys above v (unordered) and the first keys
//      equal to v in column order (a workgroup scan per tile);
//   3. a bitonic sort of the batch in LDS (64-bit keys: value, then lower
//      column) and the batch's logprobs (s - m) - log S in rank order.
// So K <= 4096 reads the row 4 times. The kernel is a fallback for large K,
// outside the one-pass budget of the main top-K kernel.
// Stash rows (same page, stash_converged_logprobs): the first pass also
// finds the argmax (lowest column at m) and its rank (the columns at m); the
// row is the argmax, then the request's token ids (gathered) or the K_out
// largest keys, then token 0 at -inf up to the width.
#include "topk_internal.h"

#include "chunk_common.h"
#include "device_common.h"
#include "device_math.h"

#include <float.h>

namespace rowstats {
namespace {

constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kTile = 4 * kWideThreads;  // columns per pass step
constexpr int kBatch = 4096;             // keys sorted in LDS at a time

// Unsigned order-preserving keys: value key (sign bit flipped) and the
// 64-bit key with 0x7FFFFFFF - column in the low word.
__device__ __forceinline__ uint32_t ukey32(float s) { return (uint32_t)key32(s) ^ 0x80000000u; }
__device__ __forceinline__ uint64_t ukey64(uint32_t k, int32_t col) {
  return ((uint64_t)k << 32) | (uint64_t)(uint32_t)(0x7FFFFFFF - col);
}
__device__ __forceinline__ float ukey_value(uint64_t k) {
  return key32_value((int32_t)((uint32_t)(k >> 32) ^ 0x80000000u));
}
__device__ __forceinline__ int32_t ukey_col(uint64_t k) {
  return 0x7FFFFFFF - (int32_t)(uint32_t)(k & 0xFFFFFFFFu);
}

constexpr int kDigitBits[3] = {11, 11, 10};  // radix digits, from the top
constexpr int kDigitShift[3] = {21, 10, 0};
constexpr int kBins = 2048;

struct WideShared {
  uint64_t keys[kBatch];
  uint32_t hist[kBins];
  double red_d[kWideWaves];
  float red_f[kWideWaves];
  uint32_t red_u[kWideWaves];
  uint32_t count;     // keys above v collected so far
  uint32_t digit;     // the bin the radix select picked
  uint32_t rank;      // rank left inside that bin
};

// Scaled values of this thread's four columns c0 .. c0 + 3 of row xrow
// (columns at or past V report `valid` false).
template <bool VEC>
__device__ __forceinline__ void load4(const float *xrow, int32_t c0, int32_t V, const Recip &rc,
                                      float tc, float (&s)[4], bool (&valid)[4]) {
  float x[4];
  if (VEC && c0 + 4 <= V) {
    const float4 q = *reinterpret_cast<const float4 *>(xrow + c0);
    x[0] = q.x;
    x[1] = q.y;
    x[2] = q.z;
    x[3] = q.w;
#pragma unroll
    for (int i = 0; i < 4; ++i) valid[i] = true;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      valid[i] = c0 + i < V;
      x[i] = valid[i] ? xrow[c0 + i] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = scale_any(x[i], rc, tc);
}

__device__ __forceinline__ float block_max(float v, WideShared &sh) {
  v = wave_max_f32(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) sh.red_f[w] = v;
  __syncthreads();
  float r = sh.red_f[0];
  for (int i = 1; i < kWideWaves; ++i) r = fmaxf(r, sh.red_f[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int32_t block_min(int32_t v, WideShared &sh) {
  v = wave_allreduce(v, MinI());
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) sh.red_u[w] = (uint32_t)v;
  __syncthreads();
  int32_t r = (int32_t)sh.red_u[0];
  for (int i = 1; i < kWideWaves; ++i) r = min(r, (int32_t)sh.red_u[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_sum(double v, WideShared &sh) {
  v = wave_allreduce(v, SumD());
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) sh.red_d[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < kWideWaves; ++i) r += sh.red_d[i];
  __syncthreads();
  return r;
}

// Exclusive prefix of v over the workgroup (thread order) and the total.
__device__ __forceinline__ uint32_t block_prefix(uint32_t v, uint32_t &total, WideShared &sh) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_up(incl, (unsigned)d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) sh.red_u[w] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int i = 0; i < kWideWaves; ++i) {
    if (i < w) off += sh.red_u[i];
    tot += sh.red_u[i];
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// The digit of the radix select from the histogram of one pass: the bin
// (from the top) where the count of higher keys first reaches `rank`, and
// the rank left inside it. Thread t scans bins nb - 1 - 2 t and nb - 2 - 2 t.
__device__ __forceinline__ void pick_digit(int nb, uint32_t rank, WideShared &sh) {
  const int t = threadIdx.x;
  const int hi = nb - 1 - 2 * t;
  const uint32_t c0 = hi >= 0 ? sh.hist[hi] : 0u;
  const uint32_t c1 = hi >= 1 ? sh.hist[hi - 1] : 0u;
  uint32_t total;
  const uint32_t before = block_prefix(c0 + c1, total, sh);  // keys in higher bins
  if (before < rank && before + c0 >= rank) {
    sh.digit = (uint32_t)hi;
    sh.rank = rank - before;
  } else if (before + c0 < rank && before + c0 + c1 >= rank) {
    sh.digit = (uint32_t)(hi - 1);
    sh.rank = rank - before - c0;
  }
  __syncthreads();
}

template <bool VEC>
__global__ __launch_bounds__(kWideThreads) void topk_wide_kernel(TopKParams p) {
  __shared__ WideShared sh;
  const int64_t pos = blockIdx.x;
  if (pos >= p.kept[p.rows]) return;
  const int t = threadIdx.x;
  const int64_t row = p.kept[pos];
  const float tc = clamp_temp(p.kept_temp[pos]);
  const Recip rc = recip_of(tc);
  const float *xrow = p.logits + row * p.ld;
  const int32_t V = p.vocab;
  constexpr float kL2e = 1.44269504088896340736f;
  int K = p.K;

  // ---- first pass: m, S (online), the stash's argmax and rank, and the
  // histogram of the first digit of every key ----
  for (int i = t; i < kBins; i += kWideThreads) sh.hist[i] = 0u;
  __syncthreads();
  float mt = -INFINITY, st = 0.0f;
  uint32_t at_max = 0;        // columns whose key is mt's (-0 == +0)
  int32_t first = INT32_MAX;  // the lowest of them
  for (int32_t base = 0; base < V; base += kTile) {
    float s[4];
    bool ok[4];
    const int32_t c0 = base + 4 * t;
    load4<VEC>(xrow, c0, V, rc, tc, s, ok);
    float m4 = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ok[i]) {
        m4 = fmaxf(m4, s[i]);
        atomicAdd(&sh.hist[ukey32(s[i]) >> kDigitShift[0]], 1u);
      }
    }
    if (m4 > mt) {
      st *= __builtin_amdgcn_exp2f(fmaxf(mt - m4, -FLT_MAX) * kL2e);
      if (p.stash && ukey32(m4) != ukey32(mt)) {
        at_max = 0;
        first = INT32_MAX;
      }
      mt = m4;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ok[i]) {
        st += __builtin_amdgcn_exp2f(fmaxf(s[i] - mt, -FLT_MAX) * kL2e);
        if (p.stash && ukey32(s[i]) == ukey32(mt)) {
          ++at_max;
          first = min(first, c0 + i);
        }
      }
    }
  }
  const float m = block_max(mt, sh);
  const uint32_t km = ukey32(m);
  const bool mine = mt != -INFINITY && ukey32(mt) == km;  // this thread's maximum is the row's
  const double part =
      mt == -INFINITY ? 0.0 : (double)st * (double)__builtin_amdgcn_exp2f(fmaxf(mt - m, -FLT_MAX) * kL2e);
  const double log_s = log_d(block_sum(part, sh));

  // stash rows: argmax, rank, token ids and padding here, the top keys below
  int32_t *oid = nullptr;
  float *olp = nullptr;
  const bool logits_mode = p.stash && p.logits_mode != 0;
  auto value = [&](float s) -> float {
    return logits_mode ? s : (float)(((double)s - (double)m) - log_s);
  };
  if (p.stash) {
    uint32_t ties;
    block_prefix(mine ? at_max : 0u, ties, sh);
    const int32_t arg = block_min(mine ? first : INT32_MAX, sh);
    const int64_t dst = p.kept_dst[pos];
    const int32_t j = p.kept_req[pos];
    const int32_t W = p.width;
    oid = p.out_ids32 + dst * W;
    olp = p.out_lp + dst * W;
    int n = p.K_out;
    bool by_ids = false;
    if (p.ids != nullptr) {
      const int32_t c = p.num_ids[j];
      if (c > 0) {
        by_ids = true;
        n = (int)min((int64_t)min(c, W - 1), p.ids_stride);
      }
    }
    if (t == 0) {
      oid[0] = arg;
      olp[0] = value(key32_value((int32_t)(km ^ 0x80000000u)));
      p.out_ranks[dst] = (int32_t)ties;
    }
    if (by_ids) {
      const int32_t *idr = p.ids + (int64_t)j * p.ids_stride;
      for (int i = t; i < n; i += kWideThreads) {
        const int32_t id = idr[i];
        float v = -INFINITY;
        if (id >= 0 && id < V) v = value(scale_any(xrow[id], rc, tc));
        else atomicOr(p.err_flag, kErrIndex);
        oid[1 + i] = id;
        olp[1 + i] = v;
      }
    }
    for (int c = 1 + n + t; c < W; c += kWideThreads) {
      oid[c] = 0;
      olp[c] = -INFINITY;
    }
    K = by_ids ? 0 : n;
  }

  // ---- batches of keys in descending order ----
  uint64_t bound = ~0ull;  // keys of this batch are below it
  bool bounded = false;
  for (int done = 0; done < K;) {
    const int nb = min(K - done, kBatch);
    auto allowed = [&](uint32_t k, int32_t c) { return !bounded || ukey64(k, c) < bound; };
    // radix select: v = value key of the nb-th largest allowed key
    uint32_t prefix = 0;
    uint32_t rank = (uint32_t)nb;  // 1-based rank from the top inside the current prefix
#pragma unroll 1
    for (int d = 0; d < 3; ++d) {
      const int shift = kDigitShift[d];
      const int bins = 1 << kDigitBits[d];
      if (d > 0 || bounded) {  // the first batch's first histogram came with m and S
        for (int i = t; i < kBins; i += kWideThreads) sh.hist[i] = 0u;
        __syncthreads();
        const int hshift = shift + kDigitBits[d];  // bits above this digit
        for (int32_t base = 0; base < V; base += kTile) {
          float s[4];
          bool ok[4];
          load4<VEC>(xrow, base + 4 * t, V, rc, tc, s, ok);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t k = ukey32(s[i]);
            const bool match = ((uint64_t)k >> hshift) == (uint64_t)prefix;
            if (ok[i] && match && allowed(k, base + 4 * t + i))
              atomicAdd(&sh.hist[(k >> shift) & (uint32_t)(bins - 1)], 1u);
          }
        }
        __syncthreads();
      }
      pick_digit(bins, rank, sh);
      prefix = (prefix << kDigitBits[d]) | sh.digit;
      rank = sh.rank;
      __syncthreads();
    }
    const uint32_t v = prefix;
    const uint32_t need = rank;  // keys equal to v that belong to the batch
    const uint32_t above = (uint32_t)nb - need;

    // one pass: the keys above v, in any order, and the first `need` keys
    // equal to v, in column order
    if (t == 0) sh.count = 0u;
    __syncthreads();
    uint32_t taken = 0;
    for (int32_t base = 0; base < V; base += kTile) {
      float s[4];
      bool ok[4];
      load4<VEC>(xrow, base + 4 * t, V, rc, tc, s, ok);
      bool tie[4];
      uint32_t ties_here = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t k = ukey32(s[i]);
        const int32_t c = base + 4 * t + i;
        const bool in = ok[i] && allowed(k, c);
        if (in && k > v) {
          const uint32_t at = atomicAdd(&sh.count, 1u);
          if (at < above) sh.keys[at] = ukey64(k, c);  // (exactly `above` such keys)
        }
        tie[i] = in && k == v;
        ties_here += tie[i] ? 1u : 0u;
      }
      if (taken < need) {  // uniform: the scan has a barrier
        uint32_t total;
        uint32_t at = taken + block_prefix(ties_here, total, sh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (tie[i]) {
            if (at < need) sh.keys[above + at] = ukey64(v, base + 4 * t + i);
            ++at;
          }
        }
        taken += total;
      }
    }
    __syncthreads();
    // pad to a power of two and sort descending
    int n2 = 64;
    while (n2 < nb) n2 <<= 1;
    for (int i = nb + t; i < n2; i += kWideThreads) sh.keys[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = t; i < n2 / 2; i += kWideThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool desc = (lo & size) == 0;
          const uint64_t a = sh.keys[lo], b = sh.keys[hi];
          if ((a < b) == desc) {
            sh.keys[lo] = b;
            sh.keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    // the batch's logprobs (or a stash row's values), in rank order
    for (int i = t; i < nb; i += kWideThreads) {
      const uint64_t k = sh.keys[i];
      const float s = ukey_value(k);
      if (p.stash) {
        oid[1 + done + i] = ukey_col(k);
        olp[1 + done + i] = value(s);
      } else {
        const int64_t o = row * (int64_t)K + done + i;
        p.out_idx[o] = ukey_col(k);
        p.out_vals[o] = (float)(((double)s - (double)m) - log_s);
      }
    }
    bound = sh.keys[nb - 1];
    bounded = true;
    done += nb;
    __syncthreads();
  }
}

}  // namespace

hipError_t topk_wide_launch(const TopKParams &p, hipStream_t stream) {
  hipError_t e = p.stash ? stash_rows_launch(p, stream) : kept_rows_launch(p, stream);
  if (e != hipSuccess) return e;
  TopKParams arg = p;
  if (p.vec_ok)
    topk_wide_kernel<true><<<dim3((unsigned)p.rows), dim3(kWideThreads), 0, stream>>>(arg);
  else
    topk_wide_kernel<false><<<dim3((unsigned)p.rows), dim3(kWideThreads), 0, stream>>>(arg);
  return hipGetLastError();
}

}  // namespace rowstats
