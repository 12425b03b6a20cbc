// Top-K logprobs of the rows of kept slots, on gfx950.
//
// Method: vLLM API page "diffusion_gemma_sampler", stash_converged_logprobs
// docstring (only kept slots' rows are read; rows are divided by their
// temperature; the K largest with ties to the lower id) and the
// _lp_topk_kernel docstring (64-bit keys: order-preserving int32 of the
// value in the high word, inverted column in the low word, so keys are
// distinct and the top-K is unique; the K largest block maxima are K
// distinct elements at or above the K-th largest block maximum, so nothing
// below it can be in the top-K).
//
// Work split. As in the row-statistics kernel, a row is cut into G slices
// held in registers by one workgroup each (every logit read once). Inside a
// slice the "blocks" of the threshold rule are the 64 lane-owned column sets
// of a wave (64 columns each, strided): the K-th largest lane maximum v_K of
// a wave bounds that wave's top-K from below, so only columns with s >= v_K
// become candidates. Candidates go to an LDS list and are ranked exactly
// (rank = number of larger keys); a wave whose list would overflow falls
// back to K rounds of exact max extraction over its registers. Wave results
// merge into the slice's top-K, which is published with the slice's
// (max, sum exp) pair; the last slice of a row to arrive merges the G
// top-K lists, forms log Z and writes the row.
#include "device_common.h"
#include "topk_internal.h"

#include <float.h>
#include <limits.h>

namespace rowstats {
namespace {

constexpr int kT = kTopKThreads;
constexpr int kWv = kT / kWave;
constexpr int kCandCap = 256;    // candidate keys per wave
constexpr int kMergeCap = 2048;  // keys ranked per round of the row merge

struct TopKShared {
  int64_t buf[kMergeCap];           // per-wave candidate lists, then the row merge
  int64_t wtop[kWv * kTopKMax];     // top-K of each wave
  int64_t tops[kTopKMax];           // top-K of the slice / running row top-K
  double red_d[kWv];
  float red_f[kWv];
  int32_t red_i[kWv];
  int32_t flag;
};

// Exact top-K of n distinct keys in LDS by rank; writes out[rank] for the
// keys of rank < K. Threads [first, first + stride) take keys in turn.
__device__ __forceinline__ void rank_select(const int64_t *keys, int n, int K, int64_t *out,
                                            int first, int stride) {
  for (int i = first; i < n; i += stride) {
    const int64_t ki = keys[i];
    int r = 0;
    for (int j = 0; j < n; ++j) r += (keys[j] > ki) ? 1 : 0;
    if (r < K) out[r] = ki;
  }
}

struct SliceRecord {
  double S;   // sum over the slice of 2^32 exp(s - m)
  float m;    // slice max of s
  int32_t pad;
  // followed by K int64 keys
};

__device__ __forceinline__ int64_t *record_keys(SliceRecord *r) {
  return reinterpret_cast<int64_t *>(reinterpret_cast<char *>(r) + 16);
}

template <int QPT, bool VEC>
__device__ void topk_slice(const TopKParams &p, int64_t row, int g, TopKShared &sh) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t V = p.vocab;
  const int K = p.K;
  const float Tc = clamp_temp(p.temps[row / p.canvas_len]);
  const double rtc = 1.0 / (double)Tc;
  const float *xrow = p.logits + row * p.ld;
  const int32_t q0 = g * (kT * QPT);

  float4 v[QPT];
  const float mt = load_scaled_slice<QPT, kT, VEC>(xrow, q0, V, rtc, v);
  const float ml = block_allreduce<kT>(mt, MaxF(), sh.red_f);
  const float mu = (ml == -INFINITY) ? 0.0f : ml;
  constexpr float kLog2e = 1.44269504088896340736f;
  float St = 0.0f;
#pragma unroll
  for (int j = 0; j < QPT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      St += __builtin_amdgcn_exp2f(fmaf(fmaxf(comp(v[j], i) - mu, -FLT_MAX), kLog2e, 32.0f));
  const double Sl = block_allreduce<kT>((double)St, SumD(), sh.red_d);

  // ---- wave threshold: K-th largest lane maximum (ties ranked by lane) ----
  float vK = -INFINITY;
  if (K <= kWave) {
    int rank = 0;
#pragma unroll
    for (int l = 0; l < kWave; ++l) {
      const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mt), l));
      rank += (o > mt || (o == mt && l < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(rank == K - 1);  // exactly one lane
    if (hit != 0)
      vK = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mt), __builtin_ctzll(hit)));
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < QPT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += (comp(v[j], i) >= vK) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  int64_t *cand = sh.buf + wave * kCandCap;
  int64_t *wtop = sh.wtop + wave * kTopKMax;
  const bool fits = total <= kCandCap;
  if (fits) {
    int off = incl - cnt;
#pragma unroll
    for (int k = 0; k < 4 * QPT; ++k) {
      const float sk = comp(v[k >> 2], k & 3);
      if (sk >= vK) cand[off++] = key64(sk, slice_col<kT>(q0, k));
    }
  }
  __syncthreads();
  if (fits) {
    rank_select(cand, total, K, wtop, lane, kWave);
  } else {
    // exact fallback: K rounds of "largest key below the previous one"
    int64_t prev = INT64_MAX;
    for (int k = 0; k < K; ++k) {
      int64_t best = INT64_MIN;
#pragma unroll
      for (int k = 0; k < 4 * QPT; ++k) {
        const int64_t key = key64(comp(v[k >> 2], k & 3), slice_col<kT>(q0, k));
        if (key < prev && key > best) best = key;
      }
      best = wave_allreduce(best, MaxI64());
      if (lane == 0) wtop[k] = best;
      prev = best;
    }
  }
  __syncthreads();
  // ---- slice top-K from the waves' top-K ----
  for (int i = tid; i < kWv * K; i += kT) {
    const int64_t ki = sh.wtop[(i / K) * kTopKMax + (i % K)];
    int r = 0;
    for (int w = 0; w < kWv; ++w)
      for (int k = 0; k < K; ++k) r += (sh.wtop[w * kTopKMax + k] > ki) ? 1 : 0;
    if (r < K) sh.tops[r] = ki;
  }
  __syncthreads();

  // ---- publish the slice record (wave 0 writes, lane 0 releases) ----
  const size_t rec_bytes = topk_partial_bytes(K);
  char *base = reinterpret_cast<char *>(p.partials) + (size_t)row * p.G * rec_bytes;
  uint32_t *ctr = p.counters + (size_t)p.parity * p.counter_stride + row;
  if (wave == 0) {
    SliceRecord *rec = reinterpret_cast<SliceRecord *>(base + (size_t)g * rec_bytes);
    if (lane < K) record_keys(rec)[lane] = sh.tops[lane];
    if (lane == 0) {
      rec->S = Sl;
      rec->m = ml;
      rec->pad = 0;
      const uint32_t old =
          __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      sh.flag = (old == (uint32_t)(p.G - 1));
    }
  }
  __syncthreads();
  const bool last = sh.flag != 0;
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- last slice of the row: merge G records ----
  float m = -INFINITY;
  for (int i = tid; i < p.G; i += kT)
    m = fmaxf(m, reinterpret_cast<const SliceRecord *>(base + (size_t)i * rec_bytes)->m);
  m = block_allreduce<kT>(m, MaxF(), sh.red_f);
  double S = 0.0;
  for (int i = tid; i < p.G; i += kT) {
    const SliceRecord *rec = reinterpret_cast<const SliceRecord *>(base + (size_t)i * rec_bytes);
    if (rec->S > 0.0) S += rec->S * exp((double)rec->m - (double)m);
  }
  S = block_allreduce<kT>(S, SumD(), sh.red_d);
  // log Z - m, with the 2^32 factor of every exp value removed; the
  // logprob is then (s - m) - logS, whose first difference is exact
  const double logS = log(S) - 32.0 * 0.69314718055994530942;

  const int total_keys = p.G * K;
  int have = 0;
  for (int pos = 0; pos < total_keys;) {
    const int chunk = min(kMergeCap - have, total_keys - pos);
    for (int i = tid; i < have; i += kT) sh.buf[i] = sh.tops[i];
    for (int i = tid; i < chunk; i += kT) {
      const int t = pos + i;
      const SliceRecord *rec =
          reinterpret_cast<const SliceRecord *>(base + (size_t)(t / K) * rec_bytes);
      sh.buf[have + i] = reinterpret_cast<const int64_t *>(reinterpret_cast<const char *>(rec) + 16)[t % K];
    }
    __syncthreads();
    rank_select(sh.buf, have + chunk, K, sh.tops, tid, kT);
    __syncthreads();
    have = K;
    pos += chunk;
  }
  if (tid < K) {
    const int64_t key = sh.tops[tid];
    const float s = key32_value((int32_t)(key >> 32));
    p.out_idx[row * K + tid] = key64_col(key);
    p.out_vals[row * K + tid] = (float)(((double)s - (double)m) - logS);
  }
}

template <int QPT, bool VEC>
__global__ __launch_bounds__(kT, 4) void topk_kernel(TopKParams p) {
  __shared__ TopKShared sh;
  const int nwg = gridDim.x;
  int L = blockIdx.x;
  if (p.xcd_map) L = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  // this call counts in bank `parity`; zero the other bank for the next call
  {
    uint32_t *other = p.counters + (size_t)(p.parity ^ 1) * p.counter_stride;
    for (int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x; i < p.counter_stride;
         i += (int64_t)nwg * kT)
      other[i] = 0u;
  }
  const int64_t items = p.rows * (int64_t)p.G;
  for (int64_t it = L; it < items; it += nwg) {
    const int64_t row = it / p.G;
    const int g = (int)(it - row * p.G);
    if (!p.keep[row / p.canvas_len]) continue;
    topk_slice<QPT, VEC>(p, row, g, sh);
  }
}

}  // namespace

static const void *topk_kernel_ptr(bool vec) {
  return vec ? reinterpret_cast<const void *>(&topk_kernel<kTopKQPT, true>)
             : reinterpret_cast<const void *>(&topk_kernel<kTopKQPT, false>);
}

hipError_t topk_resident_blocks(bool vec, int *blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, topk_kernel_ptr(vec), kT, 0);
}

hipError_t topk_launch(const TopKParams &p, int grid, hipStream_t stream) {
  TopKParams arg = p;
  void *args[] = {&arg};
  return hipLaunchKernel(topk_kernel_ptr(p.vec_ok != 0), dim3(grid), dim3(kT), args, 0, stream);
}

}  // namespace rowstats
