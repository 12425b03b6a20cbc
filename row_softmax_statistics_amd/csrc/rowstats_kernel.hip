// One-pass row statistics (argmax, Gumbel-max sample, entropy, optional
// softmax) of temperature-scaled fp32 logits on gfx950.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (each
// row is read once with an online max and sum, the noise is drawn inline and
// the probabilities are written once) and sample_row_stats /
// sample_row_stats_reference (the statistics and the greedy rule).
//
// Work split. A row of `vocab` columns is cut into G slices of
// kThreads * QPT quads (4 columns each); one workgroup owns one slice at a
// time and keeps it in registers (QPT float4 per thread), so every logit is
// read from HBM exactly once. Each workgroup reduces its slice to a partial
// tuple (max m_g, its lowest column, S_g = sum 2^32 exp(s - m_g),
// W_g = sum 2^32 exp(s - m_g) (s - m_g), best perturbed score and column)
// and publishes it to global scratch.
//   - Without probs: the last workgroup of a row to arrive (row counter)
//     merges the G tuples and writes the row's outputs.
//   - With probs: the grid is persistent and cooperative (all workgroups
//     resident); the G workgroups of a row wait for each other's tuples,
//     each merges them and rescales its own register-resident exp values
//     into probabilities, so the probs are written once and the logits are
//     never re-read.
//
// Gumbel sample. A slice's own argmax a gives a lower bound
// z_lb = s_a + g_a on the slice's best perturbed score. Any column that can
// reach z_lb needs s >= z_lb - 22.8739 (the largest Gumbel value a 32-bit
// word yields), so quads below that skip the Philox draw. A drawn column is
// scored exactly (fp64 logs) only if 1 - u <= exp(s - z_lb), which every
// column reaching z_lb satisfies because -log u >= 1 - u; that test reuses
// the column's exp value, so the logs run on a few columns per slice.
#include "device_common.h"
#include "rowstats_internal.h"

#include <float.h>
#include <limits.h>

namespace rowstats {

constexpr int kThreads = kRowThreads;
constexpr int kWaves = kThreads / kWave;
constexpr uint32_t kSpinLimit = 1u << 21;

// Merge of the G partial tuples of one row by wave 0. Results are valid in
// every lane of wave 0.
struct RowMerge {
  float m;
  double S, W;
  int32_t am;
  double zb;
  int32_t zc;
  float H;  // entropy of the row
};

__device__ __attribute__((noinline)) RowMerge merge_partials(const Partial *P, int G) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  for (int i = lane; i < G; i += kWave) m = fmaxf(m, P[i].m);
  m = wave_allreduce(m, MaxF());
  double S = 0.0, W = 0.0, zb = -INFINITY;
  int32_t am = INT_MAX;
  for (int i = lane; i < G; i += kWave) {
    const Partial q = P[i];
    if (q.S > 0.0) {
      const double dm = (double)q.m - (double)m;
      const double f = exp(dm);
      S += q.S * f;
      W += f * (q.W + q.S * dm);
    }
    if (q.m == m) am = min(am, q.am);
    zb = fmax(zb, q.zb);
  }
  RowMerge r;
  r.m = m;
  r.S = wave_allreduce(S, SumD());
  r.W = wave_allreduce(W, SumD());
  r.am = wave_allreduce(am, MinI());
  r.zb = wave_allreduce(zb, MaxD());
  int32_t zc = INT_MAX;
  for (int i = lane; i < G; i += kWave) {
    const Partial q = P[i];
    if (q.zb == r.zb) zc = min(zc, q.zc);
  }
  r.zc = wave_allreduce(zc, MinI());
  // H = log S - W / S in units where every exp value carries a 2^32 factor
  r.H = (float)(log(r.S) - r.W / r.S - 32.0 * 0.69314718055994530942);
  return r;
}

__device__ __forceinline__ void write_row_outputs(const RowStatsParams &p, int64_t row,
                                                  bool greedy, const RowMerge &r) {
  p.argmax[row] = r.am;
  p.sample[row] = greedy ? (int64_t)r.am : (int64_t)r.zc;
  p.entropy[row] = r.H;
}

// Filters of the Gumbel pass for a slice with max m and bound zlb (fp64 work
// kept out of line). A quad whose e values are all below ethr has
// s < zlb - 22.8739 on every column; a column can reach zlb only if
// 1 - u <= e * kc * 2^-32 (because -log u >= 1 - u). Both carry a 2^-10
// margin for the rounding of e.
struct GumbelFilter {
  float ethr, kc;
};
__device__ __attribute__((noinline)) GumbelFilter gumbel_filter(float ml, double zlb) {
  const double thr = zlb - kGumbelMax - fabs(zlb) * 0x1p-20;
  GumbelFilter f;
  f.ethr = (float)(exp(thr - (double)ml) * 0x1p32 * (1.0 - 0x1p-10));
  f.kc = (float)(exp((double)ml - zlb) * (1.0 + 0x1p-10));
  return f;
}
// Expected number of columns passing the 1 - u test: sum_c exp(s_c - zlb).
__device__ __attribute__((noinline)) double expected_candidates(double Sl, float ml, double zlb) {
  return Sl * 0x1p-32 * exp((double)ml - zlb);
}
// Scale turning a slice's e values into probabilities: exp(m_g - m) / S.
__device__ __attribute__((noinline)) float prob_scale(float ml, float m, double S) {
  return (ml == -INFINITY) ? 0.0f : (float)(exp((double)ml - (double)m) / S);
}

// Everything one workgroup does for slice g of `row`.
template <int QPT, int PROBS, bool VEC>
__device__ __forceinline__ void process_slice(const RowStatsParams &p, int64_t row, int g,
                                              float *lds_f, int32_t *lds_i, double *lds_d,
                                              float *lds_bc) {
  const int tid = threadIdx.x;
  const int32_t V = p.vocab;
  const float T = p.temps[row / p.canvas_len];
  const bool greedy = !(T > 0.0f);
  const float Tc = clamp_temp(T);
  const double rtc = 1.0 / (double)Tc;
  const float *xrow = p.logits + row * p.ld;
  const int32_t q0 = g * (kThreads * QPT);

  // ---- load the slice once and scale it: s = fl32(x / Tc) ----
  float4 v[QPT];
  const float mt = load_scaled_slice<QPT, kThreads, VEC>(xrow, q0, V, rtc, v);
  const float ml = block_allreduce<kThreads>(mt, MaxF(), lds_f);

  // ---- lowest column attaining the slice max ----
  int32_t amk = INT_MAX;
  if (mt == ml) {
#pragma unroll
    for (int k = 4 * QPT - 1; k >= 0; --k)
      if (comp(v[k >> 2], k & 3) == ml) amk = k;
  }
  const int32_t aml =
      block_allreduce<kThreads>(amk == INT_MAX ? INT_MAX : slice_col<kThreads>(q0, amk), MinI(),
                                lds_i);

  // ---- exp values e = 2^32 exp(s - m) in place of s, and their sums ----
  // The 2^32 factor keeps every probability that survives rounding to
  // bf16/fp16 away from fp32 denormals; it cancels in every ratio.
  const float mu = (ml == -INFINITY) ? 0.0f : ml;
  constexpr float kLog2e = 1.44269504088896340736f;
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
  const double Sl = block_allreduce<kThreads>((double)St, SumD(), lds_d);
  const double Wl = block_allreduce<kThreads>((double)Wt, SumD(), lds_d);

  // ---- Gumbel-max over the slice (T > 0) ----
  double bz = -INFINITY;
  int32_t bc = INT_MAX;
  const bool noise = !greedy && ml != -INFINITY;
  if (noise) {
    const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
    const uint32_t r0 = (uint32_t)(uint64_t)row, r1 = (uint32_t)((uint64_t)row >> 32);
    // lower bound from the slice argmax
    double zlb = (double)ml + gumbel_of_word(pick(philox4x32_10((uint32_t)(aml >> 2), 0u, r0, r1,
                                                                k0, k1), aml & 3));
    // A flat slice lets many columns pass the test below; the expected
    // number is sum_c exp(s_c - zlb). Tighten zlb with every thread's own
    // maximum when that number is large.
    if (expected_candidates(Sl, ml, zlb) > 32.0) {
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
        }
      }
      zlb = fmax(zlb, block_allreduce<kThreads>(zt, MaxD(), lds_d));
    }
    const GumbelFilter flt = gumbel_filter(ml, zlb);
    const float ethr = flt.ethr, kc = flt.kc;
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
    // exact fp64 scores of the few candidates: re-read x, redraw the word
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
  const double bzl = block_allreduce<kThreads>(bz, MaxD(), lds_d);
  const int32_t bcl = block_allreduce<kThreads>(bz == bzl ? bc : INT_MAX, MinI(), lds_i);

  // ---- publish the slice tuple ----
  Partial *P = p.partials + row * p.G;
  uint32_t *ctr = p.counters + row;
  if (tid == 0) {
    Partial t;
    t.S = Sl;
    t.W = Wl;
    t.zb = bzl;
    t.m = ml;
    t.am = aml;
    t.zc = bcl;
    t.pad = 0;
    P[g] = t;
  }

  if constexpr (PROBS == 0) {
    // last arriving workgroup merges the row
    if (tid == 0) {
      const uint32_t old =
          __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      lds_i[0] = (old == (uint32_t)(p.G - 1));
    }
    __syncthreads();
    const bool last = lds_i[0] != 0;
    __syncthreads();
    if (last && tid < kWave) {
      const RowMerge r = merge_partials(P, p.G);
      if (tid == 0) {
        write_row_outputs(p, row, greedy, r);
        __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else {
    // all G workgroups of the row are resident: wait for every tuple
    if (tid == 0) {
      __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t spins = 0;
      while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             (uint32_t)p.G) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          atomicOr(p.err_flag, 1u);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (tid < kWave) {
      const RowMerge r = merge_partials(P, p.G);
      if (tid == 0) {
        // exp value -> probability: p = e * exp(m_g - m) / S
        lds_bc[0] = prob_scale(ml, r.m, r.S);
        if (g == 0) write_row_outputs(p, row, greedy, r);
        const uint32_t old =
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(2 * p.G - 1))
          __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    const float sc = lds_bc[0];
    __syncthreads();

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
  __shared__ float lds_f[kWaves];
  __shared__ int32_t lds_i[kWaves];
  __shared__ double lds_d[kWaves];
  __shared__ float lds_bc[1];
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
      process_slice<QPT, PROBS, VEC>(p, row, g, lds_f, lds_i, lds_d, lds_bc);
    }
  } else {
    const int group = L / p.G;
    const int g = L - group * p.G;
    if (group >= p.n_groups) return;
    for (int64_t row = group; row < p.rows; row += p.n_groups)
      process_slice<QPT, PROBS, VEC>(p, row, g, lds_f, lds_i, lds_d, lds_bc);
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
