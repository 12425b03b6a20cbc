// Device helpers shared by the row-statistics and top-K kernels (gfx950,
// wave64): Philox4x32-10, exact temperature scaling, order keys, wave and
// workgroup reductions, and fp32 -> bf16/fp16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowstats {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round two 32x32->64
// products of counter words 0 and 2, xor-mixed with words 1 and 3 and the
// key; the key advances by the Weyl constants between rounds.
// Counter layout of the noise: (quad, 0, lo32(row), hi32(row)); key (seed).
// ---------------------------------------------------------------------------
struct Philox {
  static constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  static constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
};

__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += Philox::W0;
      k1 += Philox::W1;
      // Each call steps its own copy of the key in scalar registers. Without
      // the empty statement the compiler hoists all 18 round keys out of the
      // calling loop and, short of scalar registers, keeps most of them in
      // vector-register lanes, paying a vector read-lane per use.
      __asm__ volatile("" : "+s"(k0), "+s"(k1));
    }
    const uint64_t p0 = (uint64_t)Philox::M0 * c0;
    const uint64_t p1 = (uint64_t)Philox::M1 * c2;
    // three-input xor in one instruction (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  return make_uint4(c0, c1, c2, c3);
}

// The same generator with the keys of rounds 1..9 given in vector registers
// (computed once per kernel): no scalar work per call.
struct PhiloxRoundKeys {
  uint32_t a[10], b[10];
};
__device__ __forceinline__ PhiloxRoundKeys philox_round_keys_v(uint32_t k0, uint32_t k1) {
  PhiloxRoundKeys r;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t x = k0 + (uint32_t)i * Philox::W0, y = k1 + (uint32_t)i * Philox::W1;
    __asm__("v_mov_b32 %0, %1" : "=v"(r.a[i]) : "s"(x));
    __asm__("v_mov_b32 %0, %1" : "=v"(r.b[i]) : "s"(y));
  }
  return r;
}
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1,
                                               const PhiloxRoundKeys &rk) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t ka = round == 0 ? k0 : rk.a[round];
    const uint32_t kb = round == 0 ? k1 : rk.b[round];
    const uint64_t p0 = (uint64_t)Philox::M0 * c0;
    const uint64_t p1 = (uint64_t)Philox::M1 * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, ka, 0x96);
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, kb, 0x96);
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t pick(const uint4 &w, int i) {
  return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// ---------------------------------------------------------------------------
// Temperature: T <= 0 (and NaN-free T below 1e-10) clamps to 1e-10f, and
// s = fl32(x / Tc), the IEEE fp32 quotient.
//
// Fast form: s = fl32(P), P = fl64(x * fl64(1 / Tc)) = q (1 + d) with
// q = x / Tc and |d| < 2^-51.99. Write Tc = t 2^(f-23), t < 2^24 an integer.
//  * Normal results, q in [2^e, 2^(e+1)), e >= -126: a midpoint between two
//    fp32 values there is mid = (2M + 1) 2^(e-24) with 2M + 1 >= 2^24 + 1, so
//    mid Tc has more than 24 significant bits and is not x. x - mid Tc is then
//    a nonzero multiple of 2^(e+f-47), so |q - mid| > 2^(e-48) > |P - q|:
//    fl32(P) is the IEEE quotient, for every Tc.
//  * Subnormal results (|q| < 2^-126; midpoints n 2^-150, n odd) that are not
//    midpoints: x - mid Tc is a nonzero multiple of 2^min(-149, f-173), so
//    |q - mid| > 2^min(-150-f, -174) > 2^-177.99 > |P - q| when Tc < 2.
//  * A subnormal quotient equal to a midpoint n 2^-150 needs x = n 2^-150 Tc
//    to be a multiple of 2^-149, i.e. Tc = (odd) 2^k with k >= 1: Tc >= 2. It
//    happens there: x = 147 2^-149 and T = 98 give the midpoint 3 2^-150,
//    which rounds to the even 2^-148, while fl32(P) gives 2^-149.
// So scale() is exact for every x when Tc < 2.
//
// Double-double form, exact for every Tc: r_hi = fl64(1 / Tc),
// r_lo = fl64((1 - r_hi Tc) r_hi) (the residual 1 - r_hi Tc is exact in an
// fma), and P = fl64(x r_hi + fl64(x r_lo)) = q (1 + e), |e| < 2^-103.9.
// A midpoint q = n 2^-150 (or any value of at most 25 significant bits) is an
// fp64 number more than 2^-54 q from its fp64 neighbours, so P = q and the
// fp32 conversion breaks the tie to even; every other case keeps the
// distances above with a far smaller |P - q|. Rows with Tc >= 2 use it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clamp_temp(float t) { return t > 1e-10f ? t : 1e-10f; }

__device__ __forceinline__ float scale(float x, double rtc) {
  return (float)((double)x * rtc);
}

// The reciprocal of a row's clamped temperature as r_hi + r_lo.
struct Recip {
  double hi, lo;
};
__device__ __forceinline__ double uniform_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// For a wave-uniform tc the pair is moved to scalar registers, where the
// scaling loops read it without holding vector registers.
__device__ __forceinline__ Recip recip_of(float tc) {
  const double hi = 1.0 / (double)tc;
  return {hi, fma(-hi, (double)tc, 1.0) * hi};
}
__device__ __forceinline__ Recip recip_of_uniform(float tc) {
  const Recip r = recip_of(tc);
  return {uniform_f64(r.hi), uniform_f64(r.lo)};
}
__device__ __forceinline__ float scale_dd(float x, const Recip &r) {
  return (float)fma((double)x, r.hi, (double)x * r.lo);
}
// The exact quotient for any tc: the one-product form below 2, the
// double-double form from 2 on.
__device__ __forceinline__ float scale_any(float x, const Recip &r, float tc) {
  return tc < 2.0f ? scale(x, r.hi) : scale_dd(x, r);
}

// Order-preserving int32 of the fp32 bits (after +0.0f so that -0 == +0).
__device__ __forceinline__ int32_t key32(float s) {
  const int32_t b = __float_as_int(s + 0.0f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key32_value(int32_t k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}
// 64-bit key: value key in the high word, 0x7FFFFFFF - column in the low word.
__device__ __forceinline__ int64_t key64(float s, int32_t col) {
  return ((int64_t)key32(s) << 32) | (int64_t)(uint32_t)(0x7FFFFFFF - col);
}
__device__ __forceinline__ int32_t key64_col(int64_t k) {
  return 0x7FFFFFFF - (int32_t)(uint32_t)(k & 0xFFFFFFFF);
}

// ---------------------------------------------------------------------------
// float4 component access (indices are compile-time after unrolling).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max4(const float4 &a) {
  return fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
}
// Largest of four values that are all >= 0 (no NaN): the order of such fp32
// values is the order of their bit patterns.
__device__ __forceinline__ float max4_nonneg(const float4 &a) {
  const uint32_t m = max(max(__float_as_uint(a.x), __float_as_uint(a.y)),
                         max(__float_as_uint(a.z), __float_as_uint(a.w)));
  return __uint_as_float(m);
}
__device__ __forceinline__ float comp(const float4 &a, int i) {
  return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : a.w;
}
__device__ __forceinline__ void set_comp(float4 &a, int i, float v) {
  if (i == 0) a.x = v;
  else if (i == 1) a.y = v;
  else if (i == 2) a.z = v;
  else a.w = v;
}

// ---------------------------------------------------------------------------
// Buffer resources. A slice is addressed through a raw buffer descriptor
// whose base is the slice start and whose size stops at the row end: loads
// past the end return 0 and stores past it are dropped by the hardware, and
// every per-iteration offset is a constant, so no per-lane 64-bit addresses
// are kept in registers.
// ---------------------------------------------------------------------------
using Rsrc = __amdgpu_buffer_rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data, gfx9-family descriptor
constexpr int kNonTemporal = 2;         // cache policy bit: streaming store

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Scalar (uniform-address) load through the constant address space.
__device__ __forceinline__ float load_uniform(const float *p) {
  return *(const __attribute__((address_space(4))) float *)p;
}

// ---------------------------------------------------------------------------
// Rounding to the probs dtypes. p is finite and >= 0.
// ---------------------------------------------------------------------------
// Two values rounded to nearest-even and packed (a in the low half), with
// one gfx950 conversion instruction (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32;
// round-to-nearest-even is the default rounding mode, denormals are kept).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_fp16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// ---------------------------------------------------------------------------
// Wave reductions with DPP inside 16-lane rows and lane swaps across rows.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  // every lane reads a valid lane for the patterns used here; with no
  // "old" value the compiler can fold the move into the consuming operation
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
constexpr int kDppQuadSwap1 = 0xB1, kDppQuadSwap2 = 0x4E, kDppHalfMirror = 0x141,
              kDppMirror = 0x140;

__device__ __forceinline__ uint32_t xor_lanes(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

template <int STEP>
__device__ __forceinline__ uint32_t lane_exchange(uint32_t v) {
  if constexpr (STEP == 1) return dpp32<kDppQuadSwap1>(v);
  else if constexpr (STEP == 2) return dpp32<kDppQuadSwap2>(v);
  else if constexpr (STEP == 4) return dpp32<kDppHalfMirror>(v);
  else if constexpr (STEP == 8) return dpp32<kDppMirror>(v);
  else return xor_lanes(v, STEP);
}

// One reduction step across lanes STEP apart (STEP = 1..32, a power of 2):
// every lane ends with op(own, partner), partner = lane ^ STEP for STEP <= 8
// (DPP inside 16-lane rows). For 16 and 32 the gfx950 permlane swaps
// exchange whole rows / halves in the VALU: after v_permlane16_swap of two
// copies of v, one copy holds v and the other the value 16 lanes away in
// every lane (which copy is which depends on the row), so op of the two
// copies is the step's result for a commutative op.
template <int STEP, class T, class Op>
__device__ __forceinline__ T reduce_step(T v, Op op) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (STEP <= 8) {
    T o;
    if constexpr (sizeof(T) == 4) {
      o = __builtin_bit_cast(T, lane_exchange<STEP>(__builtin_bit_cast(uint32_t, v)));
    } else {
      const uint64_t b = __builtin_bit_cast(uint64_t, v);
      const uint32_t lo = lane_exchange<STEP>((uint32_t)b), hi = lane_exchange<STEP>((uint32_t)(b >> 32));
      o = __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    }
    return op(v, o);
  } else {
    auto swap = [](uint32_t x) {
      if constexpr (STEP == 16) return __builtin_amdgcn_permlane16_swap(x, x, false, false);
      else return __builtin_amdgcn_permlane32_swap(x, x, false, false);
    };
    if constexpr (sizeof(T) == 4) {
      const auto r = swap(__builtin_bit_cast(uint32_t, v));
      return op(__builtin_bit_cast(T, (uint32_t)r[0]), __builtin_bit_cast(T, (uint32_t)r[1]));
    } else {
      const uint64_t b = __builtin_bit_cast(uint64_t, v);
      const auto lo = swap((uint32_t)b), hi = swap((uint32_t)(b >> 32));
      const T a = __builtin_bit_cast(T, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]);
      const T c = __builtin_bit_cast(T, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
      return op(a, c);
    }
  }
}

// Applies `op` over groups of WIDTH lanes (WIDTH = 2..64, a power of 2);
// every lane ends with its group's result. Narrow widths reduce few items
// (the items sit in the first lanes) in fewer dependent steps.
template <int WIDTH, class T, class Op>
__device__ __forceinline__ T group_allreduce(T v, Op op) {
  if constexpr (WIDTH > 1) v = reduce_step<1>(v, op);
  if constexpr (WIDTH > 2) v = reduce_step<2>(v, op);
  if constexpr (WIDTH > 4) v = reduce_step<4>(v, op);
  if constexpr (WIDTH > 8) v = reduce_step<8>(v, op);
  if constexpr (WIDTH > 16) v = reduce_step<16>(v, op);
  if constexpr (WIDTH > 32) v = reduce_step<32>(v, op);
  return v;
}

// Applies `op` over the 64 lanes; every lane ends with the result.
template <class T, class Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
  return group_allreduce<64>(v, op);
}

struct MaxI { __device__ int32_t operator()(int32_t a, int32_t b) const { return a > b ? a : b; } };
struct MinI { __device__ int32_t operator()(int32_t a, int32_t b) const { return a < b ? a : b; } };
struct SumF { __device__ float operator()(float a, float b) const { return a + b; } };
struct SumD { __device__ double operator()(double a, double b) const { return a + b; } };
struct SumI { __device__ int32_t operator()(int32_t a, int32_t b) const { return a + b; } };
struct MaxD { __device__ double operator()(double a, double b) const { return fmax(a, b); } };
struct MaxI64 { __device__ int64_t operator()(int64_t a, int64_t b) const { return a > b ? a : b; } };

// Largest of a non-NaN fp32 value over the wave (every lane gets it), taken
// on the order-preserving integers of the bits: an fp32 max would first
// quiet (canonicalise) every value a lane exchange brings in.
__device__ __forceinline__ float wave_max_f32(float v) {
  const int32_t b = __float_as_int(v);
  const int32_t k = wave_allreduce(b ^ ((b >> 31) & 0x7FFFFFFF), MaxI());
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

}  // namespace rowstats
