// One-pass row statistics (argmax, Gumbel-max sample, entropy, optional
// softmax) of temperature-scaled fp32 logits on gfx950.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (each
// row is read once with an online max and sum, the noise is drawn inline and
// the probabilities are written once) and sample_row_stats /
// sample_row_stats_reference (the statistics and the greedy rule).
//
// Work split. A row of `vocab` columns is cut into G slices of 16384
// columns; one 512-thread workgroup owns one slice at a time and keeps it in
// registers (8 float4 per thread), so every logit is read from HBM once.
// Each wave reduces its 2048 columns on its own to a tuple
//   (m, lowest column of m, S = sum 2^32 exp(s - m),
//    W = sum 2^32 exp(s - m) (s - m), best perturbed score z, its column),
// the slice tuple is their merge, and the row tuple the merge of its G
// slice tuples, exchanged through global scratch with agent-scope atomics.
//   - Without probs: the last slice of a row to arrive merges the row and
//     writes its outputs.
//   - With probs: the grid is persistent and cooperative (all workgroups
//     resident); the G workgroups of a row wait for each other's tuples,
//     each merges them and rescales its register-resident exp values into
//     probabilities, so the probs are written once and logits never re-read.
//
// Gumbel sample (T > 0). The wave's argmax a gives a lower bound
// zlb = s_a + g_a on its best perturbed score. A column can reach zlb only
// if s >= zlb - 22.8739 (the largest Gumbel value a 32-bit word yields), so
// quads below that skip the Philox draw; a drawn column can reach zlb only
// if 1 - u <= exp(s - zlb), which follows from -log u >= 1 - u and reuses
// the column's exp value. The few columns passing both are scored exactly
// in fp64 and the best score wins (ties to the lower column).
#include "device_common.h"
#include "device_math.h"
#include "rowstats_internal.h"

#include <float.h>
#include <limits.h>

namespace rowstats {

constexpr int kThreads = kRowThreads;
constexpr int kWaves = kThreads / kWave;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr float kLog2e = 1.44269504088896340736f;
// 2^32 exp(-22.8739) = 0.49998, lowered for the 2^-13 error of -log u and
// the rounding of e: a quad whose exp values are all below kQuadSkip / a,
// a = -log u of the bound's word, cannot reach the bound.
constexpr float kQuadSkip = 0.4993f;
constexpr float kTestMargin = 1.0f + 0x1p-10f;

// A wave, slice or row summary relative to its own maximum m.
struct Tuple {
  float m;
  int32_t am;
  double S;
  double W;
  double zb;
  int32_t zc;
};

struct SliceShared {
  Tuple wave[kWaves];
  float scale[kWaves];
};

// Merge over the wave of items 0..n-1 (lane i takes i, i + 64, ...); the
// result is valid in every lane. `get(i)` returns item i.
template <class Get>
__device__ __forceinline__ Tuple merge_tuples(int n, Get get) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  for (int i = lane; i < n; i += kWave) m = fmaxf(m, get(i).m);
  m = wave_allreduce(m, MaxF());
  double S = 0.0, W = 0.0, zb = -INFINITY;
  int32_t am = INT_MAX;
  for (int i = lane; i < n; i += kWave) {
    const Tuple t = get(i);
    if (t.S > 0.0) {
      const double dm = (double)t.m - (double)m;
      const double f = exp_d(dm);
      S += t.S * f;
      W += f * (t.W + t.S * dm);
    }
    if (t.m == m) am = min(am, t.am);
    zb = fmax(zb, t.zb);
  }
  Tuple r;
  r.m = m;
  r.S = wave_allreduce(S, SumD());
  r.W = wave_allreduce(W, SumD());
  r.am = wave_allreduce(am, MinI());
  r.zb = wave_allreduce(zb, MaxD());
  int32_t zc = INT_MAX;
  for (int i = lane; i < n; i += kWave) {
    const Tuple t = get(i);
    if (t.zb == r.zb) zc = min(zc, t.zc);
  }
  r.zc = wave_allreduce(zc, MinI());
  return r;
}

// Slice tuples in global scratch: five 64-bit words written and read with
// relaxed agent-scope atomics, so each access is coherent across XCDs
// without flushing or invalidating whole caches.
constexpr int kTupleWords = kSliceTupleWords;

__device__ __forceinline__ void store_tuple_word(uint64_t *dst, int k, const Tuple &t) {
  uint64_t v;
  switch (k) {
    case 0: v = (uint64_t)__float_as_uint(t.m) | ((uint64_t)(uint32_t)t.am << 32); break;
    case 1: v = (uint64_t)__double_as_longlong(t.S); break;
    case 2: v = (uint64_t)__double_as_longlong(t.W); break;
    case 3: v = (uint64_t)__double_as_longlong(t.zb); break;
    default: v = (uint64_t)(uint32_t)t.zc; break;
  }
  __hip_atomic_store(dst + k, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Tuple load_tuple(const uint64_t *src) {
  uint64_t w[kTupleWords];
#pragma unroll
  for (int k = 0; k < kTupleWords; ++k)
    w[k] = __hip_atomic_load(const_cast<uint64_t *>(src) + k, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  Tuple t;
  t.m = __uint_as_float((uint32_t)w[0]);
  t.am = (int32_t)(uint32_t)(w[0] >> 32);
  t.S = __longlong_as_double((long long)w[1]);
  t.W = __longlong_as_double((long long)w[2]);
  t.zb = __longlong_as_double((long long)w[3]);
  t.zc = (int32_t)(uint32_t)w[4];
  return t;
}

// Publishes a slice tuple (lanes 0..4 of the calling wave store one word
// each), waits until the stores are done, then counts the slice in. Returns
// the counter value before the add, in every lane.
__device__ __forceinline__ uint32_t publish_tuple(uint64_t *dst, const Tuple &t, uint32_t *ctr) {
  const int lane = threadIdx.x & (kWave - 1);
  if (lane < kTupleWords) store_tuple_word(dst, lane, t);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (uint32_t)__shfl((int)old, 0, kWave);
}

__device__ __forceinline__ void write_row_outputs(const RowStatsParams &p, int64_t row,
                                                  bool greedy, const Tuple &r) {
  // H = log S - W / S, every exp value carrying a 2^32 factor
  const double H = log_d(r.S) - r.W / r.S - 32.0 * 0.69314718055994530942;
  p.argmax[row] = r.am;
  p.sample[row] = greedy ? (int64_t)r.am : (int64_t)r.zc;
  p.entropy[row] = (float)H;
}

// Everything one workgroup does for slice g of `row`.
template <int QPT, int PROBS, bool VEC>
__device__ __forceinline__ void process_slice(const RowStatsParams &p, int64_t row, int g,
                                              SliceShared &sh) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t V = p.vocab;
  const float T = p.temps[row / p.canvas_len];
  const bool greedy = !(T > 0.0f);
  const double rtc = 1.0 / (double)clamp_temp(T);
  const float *xrow = p.logits + row * p.ld;
  const int32_t q0 = g * (kThreads * QPT);

  // ---- load the slice once and scale it: s = fl32(x / Tc) ----
  float4 v[QPT];
  const float mt = load_scaled_slice<QPT, kThreads, VEC>(xrow, q0, V, rtc, v);
  const float mw = wave_allreduce(mt, MaxF());

  // ---- lowest column of the wave attaining its max ----
  int32_t amk = INT_MAX;
  if (mt == mw) {
#pragma unroll
    for (int k = 4 * QPT - 1; k >= 0; --k)
      if (comp(v[k >> 2], k & 3) == mw) amk = k;
  }
  const int32_t amw =
      wave_allreduce(amk == INT_MAX ? INT_MAX : slice_col<kThreads>(q0, amk), MinI());

  // ---- exp values e = 2^32 exp(s - m) in place of s, and their sums ----
  // The 2^32 factor keeps every probability that survives rounding to
  // bf16/fp16 away from fp32 denormals; it cancels in every ratio.
  const float mu = (mw == -INFINITY) ? 0.0f : mw;
  float St = 0.0f, Wt = 0.0f;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    float4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = fmaxf(comp(v[j], i) - mu, -FLT_MAX);
      const float ei = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, 32.0f));
      St += ei;
      Wt = fmaf(ei, d, Wt);
      set_comp(e, i, ei);
    }
    v[j] = e;
  }

  // ---- Gumbel-max over the wave's columns (T > 0) ----
  double bz = -INFINITY;
  int32_t bc = INT_MAX;
  if (!greedy && mw != -INFINITY) {
    const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
    const uint32_t r0 = (uint32_t)(uint64_t)row, r1 = (uint32_t)((uint64_t)row >> 32);
    // a = exp(m - zlb) = -log u of the argmax's word, zlb = m + g_argmax
    float a = neg_log_u_f32(
        pick(philox4x32_10((uint32_t)(amw >> 2), 0u, r0, r1, k0, k1), amw & 3));
    // Flat waves let many columns pass the test; the expected number is
    // sum_c exp(s_c - zlb) = a sum e / 2^32. When it is large, raise zlb to
    // the best exact score among every lane's own maximum.
    const float Sw = wave_allreduce(St, SumF());
    if (Sw * 0x1p-32f * a > 8.0f) {
      double zt = -INFINITY;
      if (mt != -INFINITY) {
        // e is monotone in s, so the first element with e == e(mt) holds mt
        const float et = __builtin_amdgcn_exp2f(fmaf(fmaxf(mt - mu, -FLT_MAX), kLog2e, 32.0f));
        int32_t kt = INT_MAX;
#pragma unroll
        for (int k = 4 * QPT - 1; k >= 0; --k)
          if (comp(v[k >> 2], k & 3) == et) kt = k;
        if (kt != INT_MAX) {
          const int32_t ct = slice_col<kThreads>(q0, kt);
          const uint4 w = philox4x32_10((uint32_t)(ct >> 2), 0u, r0, r1, k0, k1);
          zt = (double)mt + gumbel_of_word(pick(w, ct & 3));
          bz = zt;
          bc = ct;
        }
      }
      zt = wave_allreduce(zt, MaxD());
      a = fminf(a, (float)exp_d((double)mw - zt) * (1.0f + 0x1p-20f));
    }
    const float kc = a * kTestMargin;
    const float ethr = kQuadSkip / a;
    uint64_t cm = 0;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      if (max4(v[j]) >= ethr) {
        const uint32_t q = (uint32_t)(q0 + j * kThreads + tid);
        const uint4 w = philox4x32_10(q, 0u, r0, r1, k0, k1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cm |= (uint64_t)((float)(~pick(w, i)) <= comp(v[j], i) * kc) << (4 * j + i);
      }
    }
    // exact fp64 scores of the candidates: re-read x, redraw the word
    while (cm) {
      const int k = __builtin_ctzll(cm);
      cm &= cm - 1;
      const int32_t c = slice_col<kThreads>(q0, k);
      if (c < V) {
        const float s = scale(xrow[c], rtc);
        const uint4 w = philox4x32_10((uint32_t)(c >> 2), 0u, r0, r1, k0, k1);
        const double z = (double)s + gumbel_of_word(pick(w, c & 3));
        if (z > bz || (z == bz && c < bc)) {
          bz = z;
          bc = c;
        }
      }
    }
  }

  // ---- wave tuple, then the slice tuple (wave 0) ----
  {
    Tuple t;
    t.m = mw;
    t.am = amw;
    t.S = wave_allreduce((double)St, SumD());
    t.W = wave_allreduce((double)Wt, SumD());
    t.zb = wave_allreduce(bz, MaxD());
    t.zc = wave_allreduce(bz == t.zb ? bc : INT_MAX, MinI());
    if (lane == 0) sh.wave[wave] = t;
  }
  __syncthreads();
  uint64_t *P = p.partials + (row * p.G) * kTupleWords;
  uint32_t *ctr = p.counters + row;

  if constexpr (PROBS == 0) {
    if (wave == 0) {
      const Tuple st = merge_tuples(kWaves, [&](int i) { return sh.wave[i]; });
      const uint32_t old = publish_tuple(P + g * kTupleWords, st, ctr);
      if (old == (uint32_t)(p.G - 1)) {
        // last slice of the row: every tuple was stored before its count
        const Tuple r = merge_tuples(p.G, [&](int i) { return load_tuple(P + i * kTupleWords); });
        if (lane == 0) {
          write_row_outputs(p, row, greedy, r);
          __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();  // sh.wave is rewritten by the next slice
  } else {
    if (wave == 0) {
      const Tuple st = merge_tuples(kWaves, [&](int i) { return sh.wave[i]; });
      publish_tuple(P + g * kTupleWords, st, ctr);
      if (lane == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               (uint32_t)p.G) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            atomicOr(p.err_flag, 1u);
            break;
          }
        }
      }
      // the loads below are issued after lane 0 has seen every count
      const Tuple r = merge_tuples(p.G, [&](int i) { return load_tuple(P + i * kTupleWords); });
      // exp value of wave i -> probability: p = e exp(m_i - m) / S
      if (lane < kWaves) {
        const Tuple t = sh.wave[lane];
        sh.scale[lane] =
            (t.m == -INFINITY) ? 0.0f : (float)(exp_d((double)t.m - (double)r.m) / r.S);
      }
      if (lane == 0) {
        if (g == 0) write_row_outputs(p, row, greedy, r);
        const uint32_t old =
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(2 * p.G - 1))
          __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    const float sc = sh.scale[wave];
    __syncthreads();  // sh is rewritten by the next slice

    // ---- write the slice's probabilities once ----
    const int32_t c0 = 4 * q0;
    const int32_t left = V - c0;
    const Rsrc w = make_rsrc(reinterpret_cast<uint16_t *>(p.probs) + row * (int64_t)V + c0,
                             2u * (uint32_t)min(left, 4 * kThreads * QPT));
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = comp(v[j], i) * sc;
        b[i] = (PROBS == 1) ? bf16_rne_bits(pv) : fp16_rne_bits(pv);
      }
      if constexpr (VEC) {
        const u32x2 pk = {b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(pk, w, 8u * tid, 8 * j * kThreads, kNonTemporal);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b[i], w, 8u * tid,
                                                8 * j * kThreads + 2 * i, kNonTemporal);
      }
    }
  }
}

template <int QPT, int PROBS, bool VEC>
__global__ __launch_bounds__(kThreads, 4) void rowstats_kernel(RowStatsParams p) {
  __shared__ SliceShared sh;
  const int nwg = gridDim.x;
  // XCD-aware logical id: hardware workgroup b runs on XCD b % 8; logical
  // ids that share a row (consecutive ids) are placed on one XCD.
  int L = blockIdx.x;
  if (p.xcd_map) L = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  if constexpr (PROBS == 0) {
    const int64_t items = p.rows * (int64_t)p.G;
    for (int64_t it = L; it < items; it += nwg) {
      const int64_t row = it / p.G;
      const int g = (int)(it - row * p.G);
      process_slice<QPT, PROBS, VEC>(p, row, g, sh);
    }
  } else {
    const int group = L / p.G;
    const int g = L - group * p.G;
    if (group >= p.n_groups) return;
    for (int64_t row = group; row < p.rows; row += p.n_groups)
      process_slice<QPT, PROBS, VEC>(p, row, g, sh);
  }
}

// ---------------------------------------------------------------------------
// Host side: occupancy query and launch (called by the C ABI).
// ---------------------------------------------------------------------------
template <int QPT, int PROBS, bool VEC>
static const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&rowstats_kernel<QPT, PROBS, VEC>);
}

static const void *select_kernel(int probs_dtype, bool vec) {
  if (vec) {
    switch (probs_dtype) {
      case 1: return kernel_ptr<kQPT, 1, true>();
      case 2: return kernel_ptr<kQPT, 2, true>();
      default: return kernel_ptr<kQPT, 0, true>();
    }
  }
  switch (probs_dtype) {
    case 1: return kernel_ptr<kQPT, 1, false>();
    case 2: return kernel_ptr<kQPT, 2, false>();
    default: return kernel_ptr<kQPT, 0, false>();
  }
}

hipError_t rowstats_resident_blocks(int probs_dtype, bool vec, int *blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu,
                                                      select_kernel(probs_dtype, vec), kThreads, 0);
}

hipError_t rowstats_launch(const RowStatsParams &p, int probs_dtype, int grid,
                           hipStream_t stream) {
  RowStatsParams arg = p;
  void *args[] = {&arg};
  const void *k = select_kernel(probs_dtype, p.vec_ok != 0);
  if (probs_dtype != 0)
    return hipLaunchCooperativeKernel(k, dim3(grid), dim3(kThreads), args, 0, stream);
  return hipLaunchKernel(k, dim3(grid), dim3(kThreads), args, 0, stream);
}

}  // namespace rowstats
