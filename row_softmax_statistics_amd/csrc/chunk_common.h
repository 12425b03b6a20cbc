// Chunk pipeline shared by the row-statistics and top-K kernels (gfx950):
// a wave owns a chunk of 2048 columns of a row (lane l holds quads
// j * 64 + l, j < 8), copies the next chunk from HBM into its LDS buffer
// while it reduces the current one, and exchanges results with the other
// waves of the row through device-coherent words tagged with the call's
// epoch.
#pragma once

#include <stddef.h>

#include "device_common.h"
#include "rowstats_internal.h"

namespace rowstats {

constexpr int kQ = kWaveQuads;
// Cache-policy bit sc1: a device-scope coherent load or store (the CU's L1
// is bypassed and the access is coherent across XCDs).
constexpr int kDevScope = 16;
// Polls of one wait before it gives up and flags the call (about a second);
// once any wait of a call has given up, its later waits give up at once.
constexpr uint32_t kSpinLimit = 1u << 20;

typedef __attribute__((address_space(3))) void *LdsPtr;

// Lane within the wave, from mbcnt (bits of an all-ones mask below the
// lane): it needs no input register, so the compiler can recompute it
// instead of keeping threadIdx.x alive through the kernel.
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// The same, computed where it is written: the compiler cannot move volatile
// inline assembly out of a loop, so values derived from it inside a row loop
// are recomputed there instead of being kept (and spilled to scratch
// memory, whose reloads wait for the chunk copy in flight) across the loop.
__device__ __forceinline__ int lane_here() {
  uint32_t l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return (int)l;
}

// Keeps the compiler from moving memory operations across this point, so
// the counts above hold for the issue order written here.
__device__ __forceinline__ void compiler_fence() { __asm__ volatile("" ::: "memory"); }

// Exclusive prefix sum over the lanes of cnt (0 <= cnt < 128) and the wave
// total, one bit of cnt at a time: a ballot of the bit and mbcnt (set bits
// of lower lanes).
__device__ __forceinline__ int wave_prefix(int cnt, int &total) {
  int off = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint64_t m = __ballot((cnt >> b) & 1);
    off += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))
           << b;
    tot += __popcll(m) << b;
    if (__ballot(cnt >> (b + 1)) == 0) break;
  }
  total = tot;
  return off;
}

// Keeps the compiler's LDS accesses in program order between lanes of a
// wave (the hardware executes a wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  compiler_fence();
}

// ---------------------------------------------------------------------------
// Chunk transfers. Lane l holds quads j * 64 + l (j < 8) of the chunk, so
// each load instruction of the wave covers 1 KiB of contiguous logits; the
// buffer descriptor stops at the row end (loads past it read 0 and are masked
// to -inf, stores past it are dropped).
// ---------------------------------------------------------------------------
__device__ __forceinline__ Rsrc chunk_rsrc(const float *xrow, int32_t c0, int32_t V) {
  // the size is wave-uniform; readfirstlane keeps it (and the descriptor) in
  // scalar registers even where the compiler clamps it with a vector op
  const int32_t cols = __builtin_amdgcn_readfirstlane(max(min(V - c0, kChunkCols), 0));
  return make_rsrc(xrow + c0, 4u * (uint32_t)cols);
}

// Bytes of the chunk at column c0 of a row of V columns (wave-uniform).
__device__ __forceinline__ uint32_t chunk_bytes(int32_t c0, int32_t V) {
  return 4u * (uint32_t)__builtin_amdgcn_readfirstlane(max(min(V - c0, kChunkCols), 0));
}

// Cache-policy bit nt on the chunk copies: every logit is read once, so the
// copies stream past the caches (measured about 1 % faster than the default
// policy on every row-statistics workload).
constexpr int kStreamLoad = 2;

// Vector path: asynchronous copy of `bytes` bytes at src (a chunk) into the
// wave's LDS buffer (quad j * 64 + l at buf[j * 64 + l]); the rest of the
// buffer gets zeros.
__device__ __forceinline__ void chunk_copy_bytes(float4 *buf, const float *src, uint32_t bytes) {
  const Rsrc r = make_rsrc(src, bytes);
  const uint32_t voff = 16u * lane_id();
  // The instruction offset moves both the HBM address and the LDS
  // destination, so M0 (the LDS base) changes only once per chunk.
#define ROWSTATS_DMA(J)                                                                          \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(buf + ((J) >> 2) * 4 * kWave), 16, voff, \
                                           4096 * ((J) >> 2), 1024 * ((J)&3), kStreamLoad)
  ROWSTATS_DMA(0);
  ROWSTATS_DMA(1);
  ROWSTATS_DMA(2);
  ROWSTATS_DMA(3);
  ROWSTATS_DMA(4);
  ROWSTATS_DMA(5);
  ROWSTATS_DMA(6);
  ROWSTATS_DMA(7);
#undef ROWSTATS_DMA
}

// Scalar path (unaligned rows or vocab % 4 != 0): four 4-byte loads a quad.
__device__ __forceinline__ void chunk_load(float4 (&v)[kQ], const float *xrow, int32_t c0,
                                           int32_t V) {
  const Rsrc r = chunk_rsrc(xrow, c0, V);
  const uint32_t voff = 16u * lane_id();
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      set_comp(v[j], i,
               __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 16 * kWave * j + 4 * i, 0)));
}

// Read of the wave's LDS buffer, written as inline assembly (ending with its
// own lgkmcnt wait): the compiler would otherwise wait for every copy still
// in flight into LDS before the read, including the one it must overlap.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const float4 *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float4 *)p;
}

// Element i (a float) of the buffer at `buf`, with its own wait, like the
// chunk read below.
__device__ __forceinline__ float lds_read_f32(const float4 *buf, int32_t i) {
  const uint32_t a = lds_addr(buf) + 4u * (uint32_t)i;
  float r;
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a) : "memory");
  return r;
}

// Quads j * 64 + lane (j < 8) of the buffer at `buf`.
__device__ __forceinline__ void lds_read_chunk(float4 (&v)[kQ], const float4 *buf) {
  const uint32_t a = lds_addr(buf) + 16u * (uint32_t)lane_id();
  f32x4 r0, r1, r2, r3, r4, r5, r6, r7;
  __asm__ volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:1024\n"
      "ds_read_b128 %2, %8 offset:2048\n"
      "ds_read_b128 %3, %8 offset:3072\n"
      "ds_read_b128 %4, %8 offset:4096\n"
      "ds_read_b128 %5, %8 offset:5120\n"
      "ds_read_b128 %6, %8 offset:6144\n"
      "ds_read_b128 %7, %8 offset:7168\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a)
      : "memory");
  const f32x4 r[kQ] = {r0, r1, r2, r3, r4, r5, r6, r7};
#pragma unroll
  for (int j = 0; j < kQ; ++j) v[j] = make_float4(r[j][0], r[j][1], r[j][2], r[j][3]);
}

// A field of the kernel's argument block, loaded where it is used. Fields
// that only a rare path needs (the merger's outputs) would otherwise be
// loaded at the kernel start and held in scalar registers across the row
// loop, pushing hot values out to vector-register lanes. The empty
// statement keeps the offset opaque, so the load is not merged with the one
// at the start. Only for kernels whose single argument is `Params`, which
// then starts the block.
template <class T>
__device__ __forceinline__ T kernel_arg_at(uint32_t offset) {
  __asm__ volatile("" : "+s"(offset));
  const __attribute__((address_space(4))) char *base =
      (const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr();
  return *reinterpret_cast<const __attribute__((address_space(4))) T *>(base + offset);
}
#define LATE_ARG(Params, field) \
  kernel_arg_at<decltype(Params::field)>((uint32_t)offsetof(Params, field))

// cm = 2 cm + (a >= b), four times (a0 first): each compare writes VCC or a
// scalar register pair and an add takes it as the carry in (the compiler
// would spend a select and a shift instead). A carry or mask read of a
// compare's result needs two wait states after the compare on gfx950; the
// compiler adds them to its own code but not inside inline assembly, so the
// compares write VCC and two scalar register pairs in turn and every add
// reads a result written at least two instructions before it.
__device__ __forceinline__ uint32_t push4_bits_ge(uint32_t cm, float a0, float a1, float a2,
                                                  float a3, float b0, float b1, float b2,
                                                  float b3) {
  uint64_t sb, sc;
  __asm__(
      "v_cmp_ge_f32_e64 vcc, %3, %7\n\t"
      "v_cmp_ge_f32_e64 %1, %4, %8\n\t"
      "v_cmp_ge_f32_e64 %2, %5, %9\n\t"
      "v_addc_co_u32_e64 %0, vcc, %0, %0, vcc\n\t"
      "v_cmp_ge_f32_e64 vcc, %6, %10\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %1\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %2\n\t"
      "v_addc_co_u32_e64 %0, vcc, %0, %0, vcc"
      : "+v"(cm), "=&s"(sb), "=&s"(sc)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3)
      : "vcc");
  return cm;
}

// Element k (0..31) of the lane's chunk registers. A per-lane index into
// registers would go through scratch memory, so this is a tree of selects
// on the bits of k. The empty statements hand the selects register values:
// selects between two array elements would otherwise be turned back into
// one indexed load.
__device__ __forceinline__ float element_at(const float4 (&v)[kQ], uint32_t k) {
  const bool b0 = (k & 1u) != 0, b1 = (k & 2u) != 0, b2 = (k & 4u) != 0, b3 = (k & 8u) != 0,
             b4 = (k & 16u) != 0;
  float q[kQ];
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    float x = v[j].x, y = v[j].y, z = v[j].z, w = v[j].w;
    __asm__("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
    q[j] = b1 ? (b0 ? w : z) : (b0 ? y : x);
  }
  const float a0 = b2 ? q[1] : q[0], a1 = b2 ? q[3] : q[2], a2 = b2 ? q[5] : q[4],
              a3 = b2 ? q[7] : q[6];
  const float c0 = b3 ? a1 : a0, c1 = b3 ? a3 : a2;
  return b4 ? c1 : c0;
}

// ---------------------------------------------------------------------------
// Row results: two 64-bit words per row, a 32-bit payload each with the
// call's epoch in the high half, stored device-coherently by the row's
// merger and polled by the row's other waves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ Rsrc row_result_rsrc(uint64_t *rowres, int64_t row) {
  return make_rsrc(rowres + row * (kRowResultBytes / 8), (uint32_t)kRowResultBytes);
}
__device__ __forceinline__ u32x4 load_row_result(uint64_t *rowres, int64_t row) {
  return __builtin_amdgcn_raw_buffer_load_b128(row_result_rsrc(rowres, row), 0u, 0, kDevScope);
}
__device__ __forceinline__ void store_row_result(uint64_t *rowres, int64_t row, uint32_t a,
                                                 uint32_t b, uint32_t epoch) {
  const u32x4 v = {a, epoch, b, epoch};
  __builtin_amdgcn_raw_buffer_store_b128(v, row_result_rsrc(rowres, row), 0u, 0, kDevScope);
}
__device__ __forceinline__ bool row_result_ready(const u32x4 &v, uint32_t epoch) {
  return ((v[1] == epoch) & (v[3] == epoch)) != 0;
}

// Error words of a scratch area: err[0] collects report bits over calls
// (cleared by rowstats_check_device), err[1] holds the epoch of the last
// call whose bounded wait gave up. Once one wait of a call has given up,
// the call's other waits give up at once; the next call (a new epoch) waits
// normally again.
__device__ __forceinline__ bool call_failed(const uint32_t *err, uint32_t epoch) {
  return __hip_atomic_load(err + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
}
__device__ __forceinline__ void give_up(uint32_t *err, uint32_t epoch) {
  atomicOr(err, kErrWait);
  __hip_atomic_store(err + 1, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the row result of `row` (pre-loaded in v) shows `epoch`;
// returns it.
__device__ __forceinline__ u32x4 wait_row_result(uint64_t *rowres, int64_t row, u32x4 v,
                                                 uint32_t epoch, uint32_t *err_flag) {
  // the retry loop sits off the common path: a loop header there would make
  // the compiler wait for every outstanding copy before the first check
  if (!row_result_ready(v, epoch)) {
    uint32_t spins = 0;
    do {
      __builtin_amdgcn_s_sleep(1);
      v = load_row_result(rowres, row);
    } while (!row_result_ready(v, epoch) && ++spins <= kSpinLimit && !call_failed(err_flag, epoch));
    if (!row_result_ready(v, epoch) && lane_id() == 0) give_up(err_flag, epoch);
  }
  return v;
}

// ---------------------------------------------------------------------------
// Dynamic row assignment. Waves of different groups share a SIMD, and the
// issue arbiter favours the oldest wave, so with a fixed share of rows per
// group the groups finish at very different times and the last part of a
// launch runs with few waves. Instead, the first kDealAhead rows of group
// g are positions g + k G (G groups); after that, member 0 of the group
// claims each next position from a call-wide counter kDealAhead rows before
// the group needs it and posts it in the group's ring of kRingSlots slots.
// A slot holds two tagged words {position | epoch, iteration | epoch}; a
// position of -1 ends the group's rows. Claims only grow, so every position
// below the limit is taken by exactly one group.
// ---------------------------------------------------------------------------
struct RowDealer {
  uint64_t *ring;     // this group's ring
  uint32_t *counter;  // this call's claim counter (zero at the start of the call)
  int64_t limit;      // positions below it exist
  int64_t first;      // first position handed out by claims: kDealAhead G
  int64_t group, G;
  uint32_t epoch;

  __device__ __forceinline__ int64_t static_pos(int n) const {
    const int64_t q = group + (int64_t)n * G;
    return q < limit ? q : -1;
  }
  __device__ __forceinline__ Rsrc ring_rsrc() const { return make_rsrc(ring, (uint32_t)kRingBytes); }
  __device__ __forceinline__ u32x4 load_slot(int n) const {
    return __builtin_amdgcn_raw_buffer_load_b128(ring_rsrc(), 16u * (uint32_t)(n % kRingSlots), 0,
                                                 kDevScope);
  }
  __device__ __forceinline__ bool slot_ready(const u32x4 &w, int n) const {
    return ((w[1] == epoch) & (w[3] == epoch) & (w[2] == (uint32_t)n)) != 0;
  }
  // Position of iteration n from its slot w (loaded earlier), waiting for
  // the post if it is not there yet.
  __device__ __forceinline__ int64_t slot_pos(u32x4 w, int n, uint32_t *err_flag) const {
    if (!slot_ready(w, n)) {
      uint32_t spins = 0;
      do {
        __builtin_amdgcn_s_sleep(1);
        w = load_slot(n);
      } while (!slot_ready(w, n) && ++spins <= kSpinLimit && !call_failed(err_flag, epoch));
      if (!slot_ready(w, n)) {
        if (lane_id() == 0) give_up(err_flag, epoch);
        return -1;
      }
    }
    return (int64_t)(int32_t)__builtin_amdgcn_readfirstlane((int)w[0]);
  }
  // Member 0: claims one position (lane 0 holds the counter value).
  __device__ __forceinline__ uint32_t claim() const {
    uint32_t v = 0;
    if (lane_id() == 0) v = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  }
  __device__ __forceinline__ int64_t claimed_pos(uint32_t v) const {
    const int64_t q = first + (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)v);
    return q < limit ? q : -1;
  }
  __device__ __forceinline__ void post(int n, int64_t q) const {
    if (lane_id() == 0) {
      const u32x4 w = {(uint32_t)q, epoch, (uint32_t)n, epoch};
      __builtin_amdgcn_raw_buffer_store_b128(w, ring_rsrc(), 16u * (uint32_t)(n % kRingSlots), 0,
                                             kDevScope);
    }
  }
};

}  // namespace rowstats
