// Self-conditioning input of the denoise step: the softmax of each row,
// rounded to bf16 (the model dtype), times the embedding table,
//   out[r, :] = sum_v bf16(p[r, v]) E[v, :],   p = softmax(x / T) of row r,
// on gfx950 bf16 matrix cores, without writing the probabilities.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (the
// softmax is produced in the model dtype for the self-conditioning matmul).
//
// The row-statistics kernel (stats only) runs first and leaves each row's
// maximum m and 1 / S (S = sum 2^32 exp(s - m)) in its row results. This
// kernel is a GEMM [rows, vocab] x [vocab, d] whose A operand is recomputed
// from the fp32 logits in the load stage, p = 2^32 exp(s - m) (1 / S),
// rounded to bf16 exactly as the probabilities would be; E is bf16 [vocab, d].
//
// Tiling: a workgroup of 8 waves computes a 256 x 256 tile of out over one of
// 8 vocab ranges (split K); wave (wm, wn) holds 128 x 64 of it as 4 x 2 blocks
// of v_mfma_f32_32x32x16_bf16 accumulators. Per step of 32 vocab columns the
// workgroup stages P (256 x 32) and E transposed (256 x 32) in LDS (two
// buffers), the global loads of the step after next in flight. Workgroup b
// runs on XCD b % 8 (round-robin dispatch) and takes vocab range b % 8, so
// the tiles sharing a range of P run on one XCD, consecutive workgroups on it
// covering the column tiles of one row tile: the P range they share comes
// from that XCD's L2. A second kernel adds the 8 partial tiles in a fixed
// order (the result does not depend on timing).
#include "device_common.h"
#include "selfcond_internal.h"

#include <float.h>

namespace rowstats {
namespace {

constexpr int kThreads = kSelfCondThreads;  // 8 waves
constexpr int kTileM = kSelfCondTileM;      // 256 rows
constexpr int kTileN = kSelfCondTileN;      // 256 columns of E
constexpr int kStepK = kSelfCondStepK;      // vocab columns per step
constexpr int kPitch = kStepK + 8;          // LDS row pitch (bf16) of both staged tiles
constexpr float kLog2e = 1.44269504088896340736f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The load stage of one thread: 16 logits of one row (thread t: row t / 2,
// columns 16 (t % 2) ..) and 16 values of one row of E (thread t: vocab row
// t / 16, columns 16 (t % 16) ..).
struct Stage {
  float x[16];
  uint4 e[2];
};

// Per-thread constants of its P row.
struct RowConst {
  bool live;       // the row exists
  float tc;        // clamped temperature
  Recip rc;
  float m, inv_s;  // row maximum and 1 / S from the row-statistics kernel
};

template <bool VEC>
__device__ __forceinline__ void load_stage(const SelfCondParams &p, const RowConst &rcst,
                                           int64_t row, int32_t k, Stage &st, int32_t ke,
                                           int32_t ek, int32_t en) {
  // P part: columns k .. k + 15 of the row, below ke
  const float *xr = p.logits + row * p.ld + k;
  if (rcst.live && k + 16 <= ke) {
    if constexpr (VEC) {
      const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = __builtin_nontemporal_load(x4 + q);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.x[4 * q + i] = v[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) st.x[i] = xr[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) st.x[i] = (rcst.live && k + i < ke) ? xr[i] : -INFINITY;
  }
  // E part: vocab row ek, columns en .. en + 15
  if (ek < ke) {
    const uint4 *er = reinterpret_cast<const uint4 *>(p.E + (int64_t)ek * p.d + en);
    st.e[0] = er[0];
    st.e[1] = er[1];
  } else {
    st.e[0] = make_uint4(0, 0, 0, 0);
    st.e[1] = make_uint4(0, 0, 0, 0);
  }
}

// bf16 probabilities of the staged logits into the P tile, E values
// transposed into the E tile (row n holds the step's 32 vocab values of
// column n).
__device__ __forceinline__ void store_stage(const RowConst &rcst, const Stage &st, uint16_t *sP,
                                            uint16_t *sE, int t) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = st.x[2 * i + h];
      float s = rcst.tc < 2.0f ? scale(x, rcst.rc.hi) : scale_dd(x, rcst.rc);
      // p = 2^32 exp(s - m) / S; -inf logits (and masked columns) give 0
      const float d = fmaxf(s - rcst.m, -FLT_MAX);
      v[h] = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, 32.0f)) * rcst.inv_s;
    }
    w[i] = pack_bf16(v[0], v[1]);
  }
  uint4 *dstp = reinterpret_cast<uint4 *>(sP + (t >> 1) * kPitch + 16 * (t & 1));
  dstp[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dstp[1] = make_uint4(w[4], w[5], w[6], w[7]);
  const int kl = t >> 4, n0 = 16 * (t & 15);
  const uint32_t ev[8] = {st.e[0].x, st.e[0].y, st.e[0].z, st.e[0].w,
                          st.e[1].x, st.e[1].y, st.e[1].z, st.e[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sE[(n0 + 2 * i) * kPitch + kl] = (uint16_t)(ev[i] & 0xFFFFu);
    sE[(n0 + 2 * i + 1) * kPitch + kl] = (uint16_t)(ev[i] >> 16);
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads, 1) void selfcond_gemm_kernel(SelfCondParams p) {
  __shared__ __align__(16) uint16_t sP[2][kTileM * kPitch];
  __shared__ __align__(16) uint16_t sE[2][kTileN * kPitch];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  // workgroup -> (vocab range, row tile, column tile): range = XCD
  const int b = blockIdx.x;
  const int split = b & (kSelfCondSplits - 1);
  const int local = b / kSelfCondSplits;
  const int mt = local / p.n_tiles, nt = local - mt * p.n_tiles;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int32_t n0 = nt * kTileN;
  const int32_t kb = split * p.k_per_split;
  const int32_t ke = min(p.vocab, kb + p.k_per_split);
  const int steps = ke > kb ? (ke - kb + kStepK - 1) / kStepK : 0;

  // this thread's P row and its constants
  const int64_t row = m0 + (t >> 1);
  RowConst rcst;
  rcst.live = row < p.rows;
  {
    const int64_t r = rcst.live ? row : 0;
    const int64_t slot = (int64_t)(((uint64_t)(uint32_t)r * p.slot_mul) >> p.slot_shift);
    rcst.tc = clamp_temp(p.temps[slot]);
    rcst.rc = recip_of(rcst.tc);
    const uint32_t *rr = reinterpret_cast<const uint32_t *>(p.rowres) + 4 * r;
    rcst.m = __uint_as_float(rr[0]);
    rcst.inv_s = __uint_as_float(rr[2]);
  }
  const int32_t xoff = 16 * (t & 1);
  const int32_t ekl = t >> 4, en = n0 + 16 * (t & 15);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Stage st;
  if (steps > 0) {
    load_stage<VEC>(p, rcst, row, kb + xoff, st, ke, kb + ekl, en);
    store_stage(rcst, st, sP[0], sE[0], t);
    if (steps > 1) load_stage<VEC>(p, rcst, row, kb + kStepK + xoff, st, ke, kb + kStepK + ekl, en);
  }
  __syncthreads();
  for (int i = 0; i < steps; ++i) {
    const uint16_t *cP = sP[i & 1];
    const uint16_t *cE = sE[i & 1];
#pragma unroll
    for (int kk = 0; kk < kStepK; kk += 16) {
      const int kq = kk + 8 * (lane >> 5);
      bf16x8 a[4], e[2];
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
        a[bm] = *reinterpret_cast<const bf16x8 *>(cP + (128 * wm + 32 * bm + (lane & 31)) * kPitch + kq);
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
        e[bn] = *reinterpret_cast<const bf16x8 *>(cE + (64 * wn + 32 * bn + (lane & 31)) * kPitch + kq);
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int bn = 0; bn < 2; ++bn)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bm], e[bn], acc[bm][bn], 0, 0, 0);
    }
    if (i + 1 < steps) {
      store_stage(rcst, st, sP[(i + 1) & 1], sE[(i + 1) & 1], t);
      if (i + 2 < steps) {
        const int32_t k2 = kb + (i + 2) * kStepK;
        load_stage<VEC>(p, rcst, row, k2 + xoff, st, ke, k2 + ekl, en);
      }
    }
    __syncthreads();
  }

  // partial tile: register i of block (bm, bn) is row 8 (i / 4) + 4 (lane / 32)
  // + i % 4, column lane % 32 of the block
  float *out = p.partial + ((int64_t)split * p.rows) * p.d;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t r = m0 + 128 * wm + 32 * bm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int32_t c = n0 + 64 * wn + 32 * bn + (lane & 31);
        if (r < p.rows) out[r * p.d + c] = acc[bm][bn][i];
      }
}

// out = sum of the 8 partials, in range order; four columns per thread.
__global__ __launch_bounds__(256) void selfcond_reduce_kernel(const float *partial, int64_t n4,
                                                              int64_t stride4, float *out) {
  const float4 *src = reinterpret_cast<const float4 *>(partial);
  float4 *dst = reinterpret_cast<float4 *>(out);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 s = src[i];
#pragma unroll
    for (int k = 1; k < kSelfCondSplits; ++k) {
      const float4 v = src[i + k * stride4];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    dst[i] = s;
  }
}

}  // namespace

hipError_t selfcond_launch(const SelfCondParams &p, hipStream_t stream) {
  const int64_t grid = (int64_t)kSelfCondSplits * p.m_tiles * p.n_tiles;
  SelfCondParams arg = p;
  if (p.vec_ok)
    selfcond_gemm_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(arg);
  else
    selfcond_gemm_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(arg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = p.rows * (int64_t)p.d / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  selfcond_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p.partial, n4, n4,
                                                                           p.out);
  return hipGetLastError();
}

}  // namespace rowstats
