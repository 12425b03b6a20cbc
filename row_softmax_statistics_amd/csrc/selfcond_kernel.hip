// Self-conditioning input of the denoise step: the softmax of each row,
// rounded to bf16 (the model dtype), times the embedding table,
//   out[r, :] = sum_v bf16(p[r, v]) E[v, :],   p = softmax(x / T) of row r,
// on gfx950 bf16 matrix cores, without writing the probabilities.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (the
// step's probabilities, kept in the model's own dtype, are the input of the
// self-conditioning matrix product).
//
// The row-statistics kernel (stats only) runs first and leaves each row's
// maximum m and 1 / S (S = sum 2^32 exp(s - m)) in its row results. This
// kernel is a GEMM [rows, vocab] x [vocab, d] whose A operand is recomputed
// from the fp32 logits in the load stage, p = 2^32 exp(s - m) (1 / S),
// rounded to bf16 exactly as the probabilities would be; E is bf16 [vocab, d].
//
// Tiling: a workgroup of 8 waves computes a 128 x 512 tile of out over one of
// 8 vocab ranges (split K); wave (wm, wn) holds 64 x 128 of it as 2 x 4 blocks
// of v_mfma_f32_32x32x16_bf16 accumulators. The wide column tile halves the
// probabilities each workgroup recomputes per MFMA, so that the vector work
// (about 9 operations and one exp2 per logit) fits under the matrix work.
// Per step of 32 vocab columns the workgroup stages P (128 x 32) and E
// transposed (512 x 32) in LDS (two buffers), the global loads of the step
// after next in flight. The two waves of a SIMD work in opposite order (one
// does its MFMAs while the other computes probabilities). Workgroup b runs on
// XCD b % 8 (round-robin dispatch) and takes vocab range b % 8, so the tiles
// sharing a range of P run on one XCD, consecutive workgroups on it covering
// the column tiles of one row tile: the logits they share come from that
// XCD's L2 (plain loads, so that they stay there). A second kernel adds the
// 8 partial tiles in a fixed order (the result does not depend on timing).
#include "device_common.h"
#include "selfcond_internal.h"

#include <float.h>

#include <type_traits>

namespace rowstats {
namespace {

constexpr int kThreads = kSelfCondThreads;  // 8 waves
constexpr int kTileM = kSelfCondTileM;      // 128 rows
constexpr int kTileN = kSelfCondTileN;      // 512 columns of E
constexpr int kStepK = kSelfCondStepK;      // vocab columns per step
constexpr int kPitch = kStepK + 8;          // LDS row pitch (bf16) of the P tile
constexpr int kEPitch = kTileN + 32;        // LDS row pitch (bf16) of the E tile
constexpr float kLog2e = 1.44269504088896340736f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Two probabilities rounded to nearest-even in the model dtype (bf16, or fp16
// with F16), packed a in the low half.
template <bool F16>
__device__ __forceinline__ uint32_t pack_p(float a, float b) {
  const f32x2_t v = {a, b};
  if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The staged operands of one thread for one step of 32 vocab columns:
// 8 logits of its P row (thread t: row t / 4, columns 8 (t % 4) ..) and
// 8 columns of 4 rows of E (lane l of wave w: vocab rows 4 w .. 4 w + 3,
// columns 8 l .. 8 l + 7; each load instruction covers 1 KiB of one row).
struct Stage {
  float x[8];
  uint4 e[4];
};

// Per-thread constants of its P row.
struct RowConst {
  Recip rc;
  float m, inv_s;  // row maximum and 1 / S from the row-statistics kernel
};

// How a wave scales its rows' logits: every row at T = 1 (s = x), every
// clamped temperature below 2 (the fast form is exact there), or any
// (the double-double form is exact at any temperature).
enum ScaleMode { kScaleOne, kScaleFast, kScaleAny };

// Loads of a step whose 32 columns all lie below the range end.
template <bool VEC>
__device__ __forceinline__ void load_full(const float *xr, const uint16_t *er, int64_t d,
                                          Stage &st) {
  if constexpr (VEC) {
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 v = x4[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) st.x[4 * q + i] = v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) st.x[i] = xr[i];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) st.e[r] = *reinterpret_cast<const uint4 *>(er + r * d);
}

// Loads of the last, partial step: logits from column xk on, E rows from ek
// on; what lies at or beyond the range end ke reads as -inf (logits) and 0 (E).
__device__ __forceinline__ void load_tail(const float *xr, int32_t xk, const uint16_t *er,
                                          int32_t ek, int64_t d, int32_t ke, Stage &st) {
#pragma unroll
  for (int i = 0; i < 8; ++i) st.x[i] = xk + i < ke ? xr[i] : -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    st.e[r] = ek + r < ke ? *reinterpret_cast<const uint4 *>(er + r * d) : make_uint4(0, 0, 0, 0);
}

// bf16 probabilities of the staged logits into the P tile (row t / 4,
// columns 8 (t % 4) ..); the E rows into the E tile as they are (row k of
// the tile is vocab row k of the step).
template <bool F16, ScaleMode MODE>
__device__ __forceinline__ void store_stage(const RowConst &rcst, const Stage &st, uint16_t *sP,
                                            uint16_t *sE, int t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = st.x[2 * i + h];
      float s;
      if constexpr (MODE == kScaleOne) s = x;
      else if constexpr (MODE == kScaleFast) s = scale(x, rcst.rc.hi);
      else s = scale_dd(x, rcst.rc);
      // p = 2^32 exp(s - m) / S; -inf logits (and masked columns) give 0
      const float dm = fmaxf(s - rcst.m, -FLT_MAX);
      v[h] = __builtin_amdgcn_exp2f(fmaf(dm, kLog2e, 32.0f)) * rcst.inv_s;
    }
    w[i] = pack_p<F16>(v[0], v[1]);
  }
  *reinterpret_cast<uint4 *>(sP + (t >> 2) * kPitch + 8 * (t & 3)) =
      make_uint4(w[0], w[1], w[2], w[3]);
  const int lane = t & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<uint4 *>(sE + (4 * (t >> 6) + r) * kEPitch + 8 * lane) = st.e[r];
}

// The MFMA work of one step: wave (wm, wn) adds P[64 wm .., k] E[k, 128 wn ..]
// over the step's 32 columns into its 2 x 4 blocks of 32 x 32. The E
// operand (8 consecutive vocab rows of one column per lane) comes from the
// row-major E tile through the LDS transpose read: within each group of 16
// lanes, lane j names 4 consecutive elements (row j / 4, columns 4 (j % 4) ..
// of a 4 x 16 block) and receives element j % 4 of the rows named by lanes
// j / 4, 4 + j / 4, 8 + j / 4, 12 + j / 4, i.e. column j of the block.
template <bool F16>
__device__ __forceinline__ void mfma_step(const uint16_t *cP, const uint16_t *cE, int wm, int wn,
                                          int lane, f32x16 (&acc)[2][4]) {
  // this lane's element of the 4 x 16 blocks: rows 8 (lane / 32) + (lane % 16) / 4,
  // columns 16 ((lane / 16) % 2) + 4 (lane % 4)
  const uint16_t *eb = cE + (8 * (lane >> 5) + ((lane & 15) >> 2)) * kEPitch +
                       128 * wn + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int kk = 0; kk < kStepK; kk += 16) {
    const int kq = kk + 8 * (lane >> 5);
    using Op = std::conditional_t<F16, f16x8, bf16x8>;
    Op a[2], e[4];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
      a[bm] = *reinterpret_cast<const Op *>(cP + (64 * wm + 32 * bm + (lane & 31)) * kPitch + kq);
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const uint16_t *q = eb + kk * kEPitch + 32 * bn;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)(__attribute__((address_space(3))) const uint16_t *)q);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4 *)(__attribute__((address_space(3))) const uint16_t *)(q + 4 * kEPitch));
      const i16x4 both[2] = {lo, hi};
      e[bn] = __builtin_bit_cast(Op, both);
    }
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn)
        if constexpr (F16)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[bm], e[bn], acc[bm][bn], 0, 0, 0);
        else
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bm], e[bn], acc[bm][bn], 0, 0, 0);
  }
}

// The full steps of the range. Before step i the P and E tiles of step i sit
// in LDS buffer i % 2 and the loads of step i + 1 are in the stage registers.
// Step i stores those into buffer (i + 1) % 2, issues the loads of step i + 2
// (the last full step again past the end) and does the MFMA work on buffer
// i % 2; waves 0-3 do the MFMA work first, waves 4-7 last, so that the two
// waves sharing a SIMD overlap their matrix and vector work.
template <bool VEC, bool F16, ScaleMode MODE, bool MFMA_FIRST>
__device__ __forceinline__ void full_steps(int nfull, const float *xr, const uint16_t *er,
                                           int64_t d, const RowConst &rcst, Stage &st,
                                           uint16_t (*sP)[kTileM * kPitch],
                                           uint16_t (*sE)[kStepK * kEPitch], int t, int wm, int wn,
                                           f32x16 (&acc)[2][4]) {
  const int lane = t & 63;
  for (int i = 0; i < nfull; ++i) {
    const int j = min(i + 2, nfull - 1);
    if constexpr (MFMA_FIRST) mfma_step<F16>(sP[i & 1], sE[i & 1], wm, wn, lane, acc);
    store_stage<F16, MODE>(rcst, st, sP[(i + 1) & 1], sE[(i + 1) & 1], t);
    load_full<VEC>(xr + (int64_t)j * kStepK, er + (int64_t)j * kStepK * d, d, st);
    if constexpr (!MFMA_FIRST) mfma_step<F16>(sP[i & 1], sE[i & 1], wm, wn, lane, acc);
    __syncthreads();
  }
}

template <bool VEC, bool F16, ScaleMode MODE>
__device__ __forceinline__ void gemm_range(int nfull, bool tail, int32_t kb, int32_t ke,
                                           const float *xr, const uint16_t *er, int64_t d,
                                           const RowConst &rcst, uint16_t (*sP)[kTileM * kPitch],
                                           uint16_t (*sE)[kStepK * kEPitch], int t, int wm, int wn,
                                           f32x16 (&acc)[2][4]) {
  Stage st;
  if (nfull > 0) {
    load_full<VEC>(xr, er, d, st);
    store_stage<F16, MODE>(rcst, st, sP[0], sE[0], t);
    const int j = min(1, nfull - 1);
    load_full<VEC>(xr + (int64_t)j * kStepK, er + (int64_t)j * kStepK * d, d, st);
  }
  __syncthreads();
  if (t < 256)
    full_steps<VEC, F16, MODE, true>(nfull, xr, er, d, rcst, st, sP, sE, t, wm, wn, acc);
  else
    full_steps<VEC, F16, MODE, false>(nfull, xr, er, d, rcst, st, sP, sE, t, wm, wn, acc);
  if (tail) {
    const int32_t k0 = kb + nfull * kStepK;
    load_tail(xr + (int64_t)nfull * kStepK, k0 + 8 * (t & 3), er + (int64_t)nfull * kStepK * d,
              k0 + 4 * (t >> 6), d, ke, st);
    store_stage<F16, MODE>(rcst, st, sP[nfull & 1], sE[nfull & 1], t);
    __syncthreads();
    mfma_step<F16>(sP[nfull & 1], sE[nfull & 1], wm, wn, t & 63, acc);
  }
}

template <bool VEC, bool F16>
__global__ __launch_bounds__(kThreads, 1) void selfcond_gemm_kernel(SelfCondParams p) {
  __shared__ __align__(16) uint16_t sP[2][kTileM * kPitch];
  __shared__ __align__(16) uint16_t sE[2][kStepK * kEPitch];
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
  const int nfull = ke > kb ? (ke - kb) / kStepK : 0;
  const bool tail = ke > kb && (ke - kb) % kStepK != 0;

  // this thread's P row (rows past the end load the last row; their
  // products are not stored) and its constants
  const int64_t row = min(m0 + (t >> 2), p.rows - 1);
  RowConst rcst;
  float tc;
  {
    const int64_t slot = (int64_t)(((uint64_t)(uint32_t)row * p.slot_mul) >> p.slot_shift);
    tc = clamp_temp(p.temps[slot]);
    rcst.rc = recip_of(tc);
    const uint32_t *rr = reinterpret_cast<const uint32_t *>(p.rowres) + 4 * row;
    rcst.m = __uint_as_float(rr[0]);
    rcst.inv_s = __uint_as_float(rr[2]);
  }
  const float *xr = p.logits + row * p.ld + kb + 8 * (t & 3);
  // E columns of this thread; in a last tile of 256 columns the upper half
  // reads the lower half again (those products are not stored)
  int32_t en = n0 + 8 * lane;
  if (en >= p.d) en -= kTileN / 2;
  const uint16_t *er = p.E + (int64_t)(kb + 4 * wave) * p.d + en;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const bool all_one = __ballot(tc != 1.0f) == 0;
  const bool all_fast = __ballot(tc >= 2.0f) == 0;
  if (all_one)
    gemm_range<VEC, F16, kScaleOne>(nfull, tail, kb, ke, xr, er, p.d, rcst, sP, sE, t, wm, wn, acc);
  else if (all_fast)
    gemm_range<VEC, F16, kScaleFast>(nfull, tail, kb, ke, xr, er, p.d, rcst, sP, sE, t, wm, wn, acc);
  else
    gemm_range<VEC, F16, kScaleAny>(nfull, tail, kb, ke, xr, er, p.d, rcst, sP, sE, t, wm, wn, acc);

  // partial tile: register i of block (bm, bn) is row 8 (i / 4) + 4 (lane / 32)
  // + i % 4, column lane % 32 of the block
  if (n0 + 128 * wn >= p.d) return;
  float *out = p.partial + ((int64_t)split * p.rows) * p.d;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t r = m0 + 64 * wm + 32 * bm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int32_t c = n0 + 128 * wn + 32 * bn + (lane & 31);
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
  const dim3 g((unsigned)grid), b(kThreads);
  if (p.f16) {
    if (p.vec_ok) selfcond_gemm_kernel<true, true><<<g, b, 0, stream>>>(arg);
    else selfcond_gemm_kernel<false, true><<<g, b, 0, stream>>>(arg);
  } else {
    if (p.vec_ok) selfcond_gemm_kernel<true, false><<<g, b, 0, stream>>>(arg);
    else selfcond_gemm_kernel<false, false><<<g, b, 0, stream>>>(arg);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return partial_sum_launch(p.partial, p.rows, p.d, p.out, stream);
}

hipError_t partial_sum_launch(const float *partial, int64_t rows, int32_t d, float *out,
                              hipStream_t stream) {
  const int64_t n4 = rows * (int64_t)d / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  selfcond_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(partial, n4, n4, out);
  return hipGetLastError();
}

}  // namespace rowstats
