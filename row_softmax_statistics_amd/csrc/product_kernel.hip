// Self-conditioning input from given probabilities: out = P E for P the
// [rows, vocab] probabilities in the model dtype (bf16 or fp16, as the
// row-statistics kernel writes them) and E the [vocab, d] token embedding
// table in the same dtype, on gfx950 matrix cores.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (the
// step's probabilities, kept in the model's own dtype, are the input of the
// self-conditioning matrix product).
//
// E is a weight: it is packed once into the order in which the matrix cores
// take their B operand, so that every wave loads its E fragments from HBM
// straight into registers, 1 KiB per load instruction, with no pass through
// LDS and no transposition. Only P goes through LDS: a workgroup's 8 waves
// share each P tile.
//
// Packed layout: blocks of 32 vocab rows x 32 columns, block (b, j) at
// element ((b * d / 32 + j) * 1024); inside a block, element h * 512 + l * 8 + i
// is E[32 b + 16 h + 8 (l / 32) + i][32 j + l % 32] (h < 2, lane l < 64,
// i < 8): the B operand of v_mfma_f32_32x32x16_{bf16,f16} for vocab rows
// 32 b + 16 h .. and columns 32 j .., lane l holding its 8 elements. The
// table is padded with zero rows to a multiple of 128 vocab rows.
//
// Tiling: a workgroup of 8 waves computes a 128 x 512 tile of out over one of
// 8 vocab ranges (split K); wave w holds rows 0..127 x columns 64 w .. 64 w + 63
// of it as 4 x 2 blocks of 32 x 32 fp32 accumulators. Per step of 64 vocab
// rows each thread stages 32 bytes of its P row (thread t: row t / 4,
// columns 16 (t % 4) ..) into the LDS tile of the next step and loads its P
// bytes of the step after next, and each wave loads its 8 E fragments of the
// next step; then it reads its A fragments from the current LDS tile and
// issues 32 MFMAs. Workgroup b runs on XCD b % 8 (round-robin dispatch) and
// takes vocab range b % 8; on an XCD, consecutive workgroups cover the column
// tiles of one row tile, so the P rows they share come from that XCD's L2.
// A second kernel adds the 8 partial tiles in a fixed order.
#include "product_internal.h"
#include "selfcond_internal.h"

#include <type_traits>

namespace rowstats {
namespace {

static_assert(kProductSplits == kSelfCondSplits, "one partial-sum kernel serves both products");

constexpr int kThreads = kProductThreads;
constexpr int kTileM = kProductTileM;
constexpr int kTileN = kProductTileN;
constexpr int kStepK = kProductStepK;
constexpr int kKK = kStepK / 16;       // MFMA k-blocks of 16 vocab rows per step
constexpr int kAV = kStepK / 32;       // 16-byte P loads per thread per step
constexpr int kPitch = kStepK + 8;     // LDS row pitch (elements) of the P tile
constexpr int kBlockU4 = kPackBlock * kPackBlock * 2 / 16;  // 16-byte units per packed block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packing: one thread per 16-byte unit (block, half h, lane l) of the table.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_embed_kernel(const uint16_t *E, int64_t vocab,
                                                         int64_t d, int64_t units,
                                                         u32x4 *packed) {
  const int64_t ncb = d / kPackBlock;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63);
    const int h = (int)((u >> 6) & 1);
    const int64_t blk = u >> 7;
    const int64_t b = blk / ncb, j = blk - b * ncb;
    const int64_t col = kPackBlock * j + (l & 31);
    const int64_t k0 = kPackBlock * b + 16 * h + 8 * (l >> 5);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = k0 + 2 * i < vocab ? E[(k0 + 2 * i) * d + col] : 0u;
      const uint32_t hi = k0 + 2 * i + 1 < vocab ? E[(k0 + 2 * i + 1) * d + col] : 0u;
      w[i] = lo | (hi << 16);
    }
    packed[u] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// The GEMM.
// ---------------------------------------------------------------------------
// This thread's P bytes of one step: columns 16 (t % 4) .. + 15 of its row.
template <bool VEC>
__device__ __forceinline__ void load_p(const uint16_t *p, u32x4 (&a)[kAV]) {
  if constexpr (VEC) {
#pragma unroll
    for (int v = 0; v < kAV; ++v) a[v] = *reinterpret_cast<const u32x4 *>(p + 8 * v);
  } else {
#pragma unroll
    for (int v = 0; v < kAV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[v][i] = (uint32_t)p[8 * v + 2 * i] | ((uint32_t)p[8 * v + 2 * i + 1] << 16);
  }
}

// The same for the last, partial step: columns at or past ke read as 0.
__device__ __forceinline__ void load_p_tail(const uint16_t *p, int32_t k, int32_t ke,
                                            u32x4 (&a)[kAV]) {
#pragma unroll
  for (int v = 0; v < kAV; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t c = k + 8 * v + 2 * i;
      const uint32_t lo = c < ke ? p[8 * v + 2 * i] : 0u;
      const uint32_t hi = c + 1 < ke ? p[8 * v + 2 * i + 1] : 0u;
      a[v][i] = lo | (hi << 16);
    }
}

__device__ __forceinline__ void store_p(uint16_t *tile, int t, const u32x4 (&a)[kAV]) {
#pragma unroll
  for (int v = 0; v < kAV; ++v)
    *reinterpret_cast<u32x4 *>(tile + (t >> 2) * kPitch + (kStepK / 4) * (t & 3) + 8 * v) = a[v];
}

// E fragments of step s for this wave's two column blocks: k-block kk (16
// vocab rows) of column block bn is half kk % 2 of block row 2 s + kk / 2.
// eb points at this lane's unit of the range's first block row; brow is the
// number of units per block row.
__device__ __forceinline__ void load_e(const u32x4 *eb, int64_t brow, int s,
                                       u32x4 (&b)[2][kKK]) {
#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
      b[bn][kk] = eb[((int64_t)s * (kStepK / kPackBlock) + (kk >> 1)) * brow + bn * kBlockU4 +
                     (kk & 1) * 64];
}

// The MFMA work of one step: all 128 rows of the P tile times this wave's
// two column blocks. The A fragment of block bm (rows 32 bm ..) and k-block
// kk: lane l holds row 32 bm + l % 32, elements 16 kk + 8 (l / 32) .. + 7.
template <bool F16>
__device__ __forceinline__ void mfma_step(const uint16_t *tile, const u32x4 (&b)[2][kKK],
                                          int lane, f32x16 (&acc)[4][2]) {
  using Op = std::conditional_t<F16, f16x8, bf16x8>;
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    Op a[4];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
      a[bm] = *reinterpret_cast<const Op *>(tile + (32 * bm + (lane & 31)) * kPitch + 16 * kk +
                                            8 * (lane >> 5));
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn) {
        const Op e = __builtin_bit_cast(Op, b[bn][kk]);
        if constexpr (F16)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[bm], e, acc[bm][bn], 0, 0, 0);
        else
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bm], e, acc[bm][bn], 0, 0, 0);
      }
  }
}

// The full steps of the range. Before step i the P tile of step i sits in
// LDS buffer i % 2, the P loads of step i + 1 in `ast` and the E fragments of
// step i in the register set of parity i. Step i stores `ast` into buffer
// (i + 1) % 2, loads the P of step i + 2 and the E of step i + 1 (the last
// full step again past the end) and does the MFMA work of step i; waves 0-3
// do their MFMAs first, waves 4-7 last, so that the two waves of a SIMD do
// not reach their loads and their matrix work at the same time.
template <bool VEC, bool F16, bool MFMA_FIRST>
__device__ __forceinline__ void full_steps(int nfull, const uint16_t *pr, const u32x4 *eb,
                                           int64_t brow, uint16_t (*tiles)[kTileM * kPitch],
                                           int t, int lane, u32x4 (&ast)[kAV],
                                           u32x4 (&b0)[2][kKK], u32x4 (&b1)[2][kKK],
                                           f32x16 (&acc)[4][2]) {
  auto step = [&](int i, u32x4 (&cur)[2][kKK], u32x4 (&nxt)[2][kKK]) {
    const int j1 = min(i + 1, nfull - 1), j2 = min(i + 2, nfull - 1);
    if constexpr (MFMA_FIRST) mfma_step<F16>(tiles[i & 1], cur, lane, acc);
    store_p(tiles[(i + 1) & 1], t, ast);
    load_p<VEC>(pr + (int64_t)j2 * kStepK, ast);
    load_e(eb, brow, j1, nxt);
    if constexpr (!MFMA_FIRST) mfma_step<F16>(tiles[i & 1], cur, lane, acc);
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < nfull; i += 2) {
    step(i, b0, b1);
    step(i + 1, b1, b0);
  }
  if (i < nfull) step(i, b0, b1);
}

template <bool VEC, bool F16>
__global__ __launch_bounds__(kThreads, 1) void product_gemm_kernel(ProductParams p) {
  __shared__ __align__(16) uint16_t tiles[2][kTileM * kPitch];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;

  // workgroup -> (vocab range, row tile, column tile): range = XCD
  const int bid = blockIdx.x;
  const int split = bid & (kProductSplits - 1);
  const int local = bid / kProductSplits;
  const int mt = local / p.n_tiles, nt = local - mt * p.n_tiles;
  const int64_t m0 = (int64_t)mt * kTileM;
  const int32_t n0 = nt * kTileN;
  const int32_t kb = split * p.k_per_split;
  const int32_t ke = min(p.vocab, kb + p.k_per_split);
  const int nfull = ke > kb ? (ke - kb) / kStepK : 0;
  const bool tail = ke > kb && (ke - kb) % kStepK != 0;

  // this thread's P row (rows past the end load the last row; their
  // products are not stored)
  const int64_t row = min(m0 + (t >> 2), p.rows - 1);
  const uint16_t *pr = p.P + row * p.ldp + kb + (kStepK / 4) * (t & 3);
  // this wave's column blocks; in a last tile of 256 columns the upper
  // waves read the lower half again (those products are not stored)
  int32_t c0 = n0 + 64 * wave;
  if (c0 >= p.d) c0 -= kTileN / 2;
  const int64_t brow = (int64_t)(p.d / kPackBlock) * kBlockU4;
  const u32x4 *eb = reinterpret_cast<const u32x4 *>(p.packed) +
                    (int64_t)(kb / kPackBlock) * brow + (c0 / kPackBlock) * kBlockU4 + lane;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  u32x4 ast[kAV];
  u32x4 b0[2][kKK], b1[2][kKK];
  if (nfull > 0) {
    load_p<VEC>(pr, ast);
    store_p(tiles[0], t, ast);
    load_p<VEC>(pr + (int64_t)min(1, nfull - 1) * kStepK, ast);
    load_e(eb, brow, 0, b0);
  }
  __syncthreads();
  if (t < kThreads / 2)
    full_steps<VEC, F16, true>(nfull, pr, eb, brow, tiles, t, lane, ast, b0, b1, acc);
  else
    full_steps<VEC, F16, false>(nfull, pr, eb, brow, tiles, t, lane, ast, b0, b1, acc);
  if (tail) {
    // the E rows past vocab are zero in the packed table; the P columns at
    // or past the range end read as 0
    const int32_t k = kb + nfull * kStepK + (kStepK / 4) * (t & 3);
    load_p_tail(pr + (int64_t)nfull * kStepK, k, ke, ast);
    store_p(tiles[nfull & 1], t, ast);
    load_e(eb, brow, nfull, b0);
    __syncthreads();
    mfma_step<F16>(tiles[nfull & 1], b0, lane, acc);
  }

  // partial tile: register i of block (bm, bn) is row 8 (i / 4) + 4 (lane / 32)
  // + i % 4, column lane % 32 of the block
  if (n0 + 64 * wave >= p.d) return;
  float *out = p.partial + ((int64_t)split * p.rows) * p.d;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t r = m0 + 32 * bm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int32_t c = n0 + 64 * wave + 32 * bn + (lane & 31);
        if (r < p.rows) out[r * p.d + c] = acc[bm][bn][i];
      }
}

}  // namespace

hipError_t pack_embed_launch(const uint16_t *E, int64_t vocab, int64_t d, uint16_t *packed,
                             hipStream_t stream) {
  const int64_t units = packed_embed_bytes(vocab, d) / 16;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  pack_embed_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      E, vocab, d, units, reinterpret_cast<u32x4 *>(packed));
  return hipGetLastError();
}

hipError_t product_launch(const ProductParams &p, hipStream_t stream) {
  const int64_t grid = (int64_t)kProductSplits * p.m_tiles * p.n_tiles;
  ProductParams arg = p;
  const dim3 g((unsigned)grid), b(kThreads);
  if (p.f16) {
    if (p.vec_ok) product_gemm_kernel<true, true><<<g, b, 0, stream>>>(arg);
    else product_gemm_kernel<false, true><<<g, b, 0, stream>>>(arg);
  } else {
    if (p.vec_ok) product_gemm_kernel<true, false><<<g, b, 0, stream>>>(arg);
    else product_gemm_kernel<false, false><<<g, b, 0, stream>>>(arg);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return partial_sum_launch(p.partial, p.rows, p.d, p.out, stream);
}

}  // namespace rowstats
