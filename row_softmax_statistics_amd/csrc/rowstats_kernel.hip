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

// Merge of items 0..n-1 of a wave (lane i takes i, i + 64, ...; n <= WIDTH
// unless WIDTH is 64). The result is valid in every lane of the first WIDTH.
// The factors exp(m_i - m) are fp32 (relative error near 1e-7); the sums
// stay fp64.
template <int WIDTH, class Get>
__device__ __forceinline__ Tuple merge_tuples(int n, Get get) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  for (int i = lane; i < n; i += kWave) m = fmaxf(m, get(i).m);
  m = group_allreduce<WIDTH>(m, MaxF());
  double S = 0.0, W = 0.0, zb = -INFINITY;
  int32_t am = INT_MAX;
  for (int i = lane; i < n; i += kWave) {
    const Tuple t = get(i);
    if (t.S > 0.0) {
      const float dm = fmaxf(t.m - m, -FLT_MAX);  // <= 0, exact when the maxima are close
      const double f = (double)__builtin_amdgcn_exp2f(dm * kLog2e);
      S += t.S * f;
      W += f * (t.W + t.S * (double)dm);
    }
    if (t.m == m) am = min(am, t.am);
    zb = fmax(zb, t.zb);
  }
  Tuple r;
  r.m = m;
  r.S = group_allreduce<WIDTH>(S, SumD());
  r.W = group_allreduce<WIDTH>(W, SumD());
  r.am = group_allreduce<WIDTH>(am, MinI());
  r.zb = group_allreduce<WIDTH>(zb, MaxD());
  int32_t zc = INT_MAX;
  for (int i = lane; i < n; i += kWave) {
    const Tuple t = get(i);
    if (t.zb == r.zb) zc = min(zc, t.zc);
  }
  r.zc = group_allreduce<WIDTH>(zc, MinI());
  return r;
}

// Row merge of G slice tuples with the narrowest lane width that holds them.
template <class Get>
__device__ __forceinline__ Tuple merge_slices(int G, Get get) {
  if (G <= 8) return merge_tuples<8>(G, get);
  if (G <= 16) return merge_tuples<16>(G, get);
  if (G <= 32) return merge_tuples<32>(G, get);
  return merge_tuples<64>(G, get);
}

// Slice tuples in global scratch, five 64-bit words each, and one counter
// per row. Two coherence modes:
//   XCD-local (p.l2_sync): every workgroup of a row runs on one XCD (the
//     launch places them so and each workgroup checks its XCC id), so the
//     XCD's L2 is their point of coherence: stores write through L1 into
//     L2, atomics execute in L2 (the counter is polled with an atomic), and
//     a reader invalidates its CU's L1 before loading tuples. Round trips
//     stay on-chip instead of queueing behind the HBM stream.
//   agent: relaxed agent-scope atomics, each coherent across XCDs on its own.
// Either way a writer waits for its stores before counting the slice in.
constexpr int kTupleWords = kSliceTupleWords;
constexpr int kL1Bypass = 1;  // sc0 cache-policy bit

struct SyncScratch {
  Rsrc tuples, counters;
  uint64_t *tuple_ptr;
  uint32_t *counter_ptr;
  bool l2;
};

__device__ __forceinline__ SyncScratch sync_scratch(const RowStatsParams &p) {
  SyncScratch s;
  s.tuple_ptr = p.partials;
  s.tuples = make_rsrc(p.partials, (uint32_t)(p.rows * p.G * kTupleWords * 8));
  s.counters = make_rsrc(p.counters + (size_t)p.parity * p.counter_stride, (uint32_t)(p.rows * 4));
  s.counter_ptr = p.counters + (size_t)p.parity * p.counter_stride;
  s.l2 = p.l2_sync != 0;
  return s;
}

__device__ __forceinline__ uint64_t tuple_word(const Tuple &t, int k) {
  switch (k) {
    case 0: return (uint64_t)__float_as_uint(t.m) | ((uint64_t)(uint32_t)t.am << 32);
    case 1: return (uint64_t)__double_as_longlong(t.S);
    case 2: return (uint64_t)__double_as_longlong(t.W);
    case 3: return (uint64_t)__double_as_longlong(t.zb);
    default: return (uint64_t)(uint32_t)t.zc;
  }
}

// word index of tuple (row, g), word k
__device__ __forceinline__ uint32_t tuple_index(const RowStatsParams &p, int64_t row, int g, int k) {
  return (uint32_t)((row * p.G + g) * kTupleWords + k);
}

// Drops this CU's L1 lines so that later loads read the XCD's L2.
__device__ __forceinline__ void l1_invalidate(const SyncScratch &s) {
  if (s.l2) __asm__ volatile("buffer_inv sc0" ::: "memory");
}

__device__ __forceinline__ Tuple load_tuple(const SyncScratch &s, uint32_t w0) {
  uint64_t w[kTupleWords];
#pragma unroll
  for (int k = 0; k < kTupleWords; ++k) {
    if (s.l2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(s.tuples, 8u * (w0 + k), 0, kL1Bypass);
      w[k] = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
    } else {
      w[k] = __hip_atomic_load(s.tuple_ptr + w0 + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  Tuple t;
  t.m = __uint_as_float((uint32_t)w[0]);
  t.am = (int32_t)(uint32_t)(w[0] >> 32);
  t.S = __longlong_as_double((long long)w[1]);
  t.W = __longlong_as_double((long long)w[2]);
  t.zb = __longlong_as_double((long long)w[3]);
  t.zc = (int32_t)(uint32_t)w[4];
  return t;
}

__device__ __forceinline__ uint32_t counter_add(const SyncScratch &s, int64_t row) {
  if (s.l2) return (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, s.counters, 4u * (uint32_t)row, 0, 0);
  return __hip_atomic_fetch_add(s.counter_ptr + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t counter_load(const SyncScratch &s, int64_t row) {
  if (s.l2) {
    // add an opaque zero: an add of a known 0 would be folded into a load,
    // which may hit a stale L1 line; the atomic always reads the L2
    uint32_t zero = 0;
    __asm__ volatile("" : "+v"(zero));
    return __hip_atomic_fetch_add(s.counter_ptr + row, zero, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  return __hip_atomic_load(s.counter_ptr + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes a slice tuple (lanes 0..4 of the calling wave store one word
// each), waits until the stores are done, then counts the slice in. Returns
// the counter value before the add, in every lane.
__device__ __forceinline__ uint32_t publish_tuple(const SyncScratch &s, uint32_t w0, const Tuple &t,
                                                  int64_t row) {
  const int lane = threadIdx.x & (kWave - 1);
  if (lane < kTupleWords) {
    const uint64_t v = tuple_word(t, lane);
    if (s.l2) {
      const u32x2 pk = {(uint32_t)v, (uint32_t)(v >> 32)};
      __builtin_amdgcn_raw_buffer_store_b64(pk, s.tuples, 8u * (w0 + lane), 0, 0);
    } else {
      __hip_atomic_store(s.tuple_ptr + w0 + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t old = 0;
  if (lane == 0) old = counter_add(s, row);
  return (uint32_t)__shfl((int)old, 0, kWave);
}

// XCC (XCD) id of the executing workgroup.
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11));  // HW_REG_XCC_ID[3:0]
}

__device__ __forceinline__ void write_row_outputs(const RowStatsParams &p, int64_t row,
                                                  bool greedy, const Tuple &r) {
  // H = log S - W / S, every exp value carrying a 2^32 factor
  const double H = log_d(r.S) - r.W / r.S - 32.0 * 0.69314718055994530942;
  p.argmax[row] = r.am;
  p.sample[row] = greedy ? (int64_t)r.am : (int64_t)r.zc;
  p.entropy[row] = (float)H;
}

// Everything one workgroup does for slice g of `row`. On entry v holds the
// slice's raw logits; `stage` (vector path) still holds them too and is
// refilled with the next slice (`next_xrow`, `next_q0`) once no wave reads
// it any more.
template <int QPT, int PROBS, bool VEC>
__device__ __forceinline__ void process_slice(const RowStatsParams &p, int64_t row, int g,
                                              SliceShared &sh, float4 (&v)[QPT], float4 *stage,
                                              const float *next_xrow, int32_t next_q0) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t V = p.vocab;
  const float T = load_uniform(p.temps + row / p.canvas_len);
  const bool greedy = !(T > 0.0f);
  const double rtc = 1.0 / (double)clamp_temp(T);
  const float *xrow = p.logits + row * p.ld;
  const int32_t q0 = g * (kThreads * QPT);

  // ---- scale the slice: s = fl32(x / Tc) ----
  const float mt = scale_slice<QPT, kThreads>(v, q0, V, rtc);
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
    // raw logit of element k of this thread (re-read, never kept in registers)
    auto raw_x = [&](int k) -> float {
      if constexpr (VEC) return comp(stage[(k >> 2) * kThreads + tid], k & 3);
      else return xrow[slice_col<kThreads>(q0, k)];
    };
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
    // Candidates in two rounds: an fp32 score relative to m (error below
    // 1e-3: s - m is exact for every candidate, -log of -log u is off by at
    // most 2^-12) picks those within 2^-8 of the wave's best, and only
    // those get the exact fp64 score.
    float za = -INFINITY;
    for (uint64_t c2 = cm; c2; c2 &= c2 - 1) {
      const int k = __builtin_ctzll(c2);
      const int32_t c = slice_col<kThreads>(q0, k);
      if (c < V) {
        const float d = scale(raw_x(k), rtc) - mw;
        const uint4 w = philox4x32_10((uint32_t)(c >> 2), 0u, r0, r1, k0, k1);
        const float ga = -__builtin_amdgcn_logf(neg_log_u_f32(pick(w, c & 3))) *
                         0.693147180559945309f;
        za = fmaxf(za, d + ga);
      }
    }
    const float zcut = wave_allreduce(za, MaxF()) - 0x1p-8f;
    for (; cm; cm &= cm - 1) {
      const int k = __builtin_ctzll(cm);
      const int32_t c = slice_col<kThreads>(q0, k);
      if (c < V) {
        const float s = scale(raw_x(k), rtc);
        const uint4 w = philox4x32_10((uint32_t)(c >> 2), 0u, r0, r1, k0, k1);
        const uint32_t wc = pick(w, c & 3);
        const float ga = -__builtin_amdgcn_logf(neg_log_u_f32(wc)) * 0.693147180559945309f;
        if ((s - mw) + ga >= zcut) {
          const double z = (double)s + gumbel_of_word(wc);
          if (z > bz || (z == bz && c < bc)) {
            bz = z;
            bc = c;
          }
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
  // no wave reads the stage any more: start copying the next slice
  if constexpr (VEC) {
    if (next_xrow) stage_slice_async<QPT, kThreads>(stage, next_xrow, next_q0, V);
  }
  const SyncScratch sy = sync_scratch(p);
  const uint32_t w_row = tuple_index(p, row, 0, 0);

  if constexpr (PROBS == 0) {
    if (wave == 0) {
      const Tuple st = merge_tuples<kWaves>(kWaves, [&](int i) { return sh.wave[i]; });
      const uint32_t old = publish_tuple(sy, w_row + g * kTupleWords, st, row);
      if (old == (uint32_t)(p.G - 1)) {
        // last slice of the row: every tuple was stored before its count
        l1_invalidate(sy);
        const Tuple r =
            merge_slices(p.G, [&](int i) { return load_tuple(sy, w_row + i * kTupleWords); });
        if (lane == 0) write_row_outputs(p, row, greedy, r);
      }
    }
  } else {
    if (wave == 0) {
      const Tuple st = merge_tuples<kWaves>(kWaves, [&](int i) { return sh.wave[i]; });
      publish_tuple(sy, w_row + g * kTupleWords, st, row);
      if (lane == 0) {
        uint32_t spins = 0;
        while (counter_load(sy, row) < (uint32_t)p.G) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            atomicOr(p.err_flag, 1u);
            break;
          }
        }
      }
      // the loads below are issued after lane 0 has seen every count
      l1_invalidate(sy);
      const Tuple r =
          merge_slices(p.G, [&](int i) { return load_tuple(sy, w_row + i * kTupleWords); });
      // exp value of wave i -> probability: p = e exp(m_i - m) / S
      if (lane < kWaves) {
        const Tuple t = sh.wave[lane];
        sh.scale[lane] = (t.m == -INFINITY)
                             ? 0.0f
                             : (float)((double)__builtin_amdgcn_exp2f(fmaxf(t.m - r.m, -FLT_MAX) * kLog2e) / r.S);
      }
      if (lane == 0 && g == 0) write_row_outputs(p, row, greedy, r);
    }
    __syncthreads();
    const float sc = sh.scale[wave];

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
  __syncthreads();  // sh is rewritten by the next slice
}

// Slice items of one workgroup: linear item index row * G + g.
struct ItemCursor {
  int64_t it, step, end;
};

template <int QPT, int PROBS, bool VEC>
__global__ __launch_bounds__(kThreads, 4) void rowstats_kernel(RowStatsParams p) {
  __shared__ SliceShared sh;
  // LDS stage of the slice (vector path): the next slice's HBM copies run
  // while the current one waits for its row and writes its probs.
  __shared__ float4 stage[VEC ? kThreads * QPT : 1];
  const int nwg = gridDim.x;
  // XCD-aware logical id: hardware workgroup b runs on XCD b % 8; logical
  // ids that share a row (consecutive ids) are placed on one XCD.
  int L = blockIdx.x;
  if (p.xcd_map) L = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  // Row counters come in two banks used by alternate calls: this call counts
  // in bank `parity` (zeroed by the previous call) and zeroes the other one
  // for the next call, so no counter is ever reset while in use.
  {
    uint32_t *other = p.counters + (size_t)(p.parity ^ 1) * p.counter_stride;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.counter_stride;
         i += (int64_t)nwg * kThreads)
      other[i] = 0u;
  }
  // XCD-local synchronisation relies on workgroup b running on XCC b % 8
  if (p.l2_sync && threadIdx.x == 0 && xcc_id() != blockIdx.x % 8) atomicOr(p.err_flag, 2u);
  // Items: without probs, linear items L, L + nwg, ...; with probs, slice g
  // of rows group, group + n_groups, ...
  ItemCursor cur;
  if constexpr (PROBS == 0) {
    cur = {L, nwg, p.rows * (int64_t)p.G};
  } else {
    const int group = L / p.G;
    if (group >= p.n_groups) return;
    cur = {(int64_t)group * p.G + (L - group * p.G), (int64_t)p.n_groups * p.G,
           p.rows * (int64_t)p.G};
  }
  if (cur.it >= cur.end) return;
  constexpr int32_t span = kThreads * QPT;
  if constexpr (VEC) {
    const int64_t row = cur.it / p.G;
    stage_slice_async<QPT, kThreads>(stage, p.logits + row * p.ld,
                                     (int32_t)(cur.it - row * p.G) * span, p.vocab);
  }
  for (; cur.it < cur.end; cur.it += cur.step) {
    const int64_t row = cur.it / p.G;
    const int g = (int)(cur.it - row * p.G);
    float4 v[QPT];
    const float *next_xrow = nullptr;
    int32_t next_q0 = 0;
    if constexpr (VEC) {
      stage_wait();
      __syncthreads();
      read_stage<QPT, kThreads>(stage, v);
      const int64_t nx = cur.it + cur.step;
      if (nx < cur.end) {
        const int64_t nrow = nx / p.G;
        next_xrow = p.logits + nrow * p.ld;
        next_q0 = (int32_t)(nx - nrow * p.G) * span;
      }
    } else {
      load_slice<QPT, kThreads, VEC>(p.logits + row * p.ld, g * span, p.vocab, v);
    }
    process_slice<QPT, PROBS, VEC>(p, row, g, sh, v, stage, next_xrow, next_q0);
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
