// Top-K logprobs of the rows of kept slots, on gfx950.
//
// Method: vLLM API page "diffusion_gemma_sampler", stash_converged_logprobs
// docstring (only kept slots' rows are read; rows are divided by their
// temperature; the K largest with ties to the lower id) and the
// _lp_topk_kernel docstring (64-bit keys: order-preserving int32 of the
// value in the high word, inverted column in the low word, so keys are
// distinct and the top-K is unique; the maxima of K different blocks are
// K different elements, none below the K-th largest block maximum t, so no
// element under t belongs to the top-K).
//
// Work split. A small pre-pass writes the list of kept rows. Then, as in
// the row-statistics kernel, a group of C member waves reduces one kept row
// at a time, one chunk of 2048 columns per wave, with the next chunk copied
// into the wave's LDS buffer while the current one is reduced; each logit
// of a kept row is read from HBM once and rows of other slots not at all.
//
// A wave reduces its chunk to a record: (m, S = sum exp(s - m)) and the
// chunk's K largest keys in rank order. The blocks of the threshold rule
// are the 64 lanes (32 columns each): with v_K the K-th largest lane
// maximum, only columns with s >= v_K can be in the chunk's top-K (about
// K + a few on typical rows). For K above 32, where the K-th largest of 64
// lane maxima falls deep into the chunk, v_K is the K-th largest of the
// lanes' two largest values instead (again K distinct columns reach it).
// The candidates are listed in LDS and ranked exactly (rank = number of
// larger keys). A chunk where the rule leaves too many columns (long runs
// of equal values) takes K rounds of exact extraction.
//
// One member per row (the merger, rotating) reads the row's C records one
// row later: the headers give log Z; the K-th largest of the lanes' largest
// chunk maxima is again a lower bound of the row's K-th key, and since each
// record is sorted, a record is read slot by slot only while its keys stay
// at or above that bound. The keys read are ranked in LDS together with the
// running top-K. The merger writes the row's logprobs and a row result that
// keeps the members in step (as in the row-statistics kernel).
#include "chunk_common.h"
#include "device_common.h"
#include "device_math.h"
#include "topk_internal.h"

#include <float.h>
#include <limits.h>

namespace rowstats {
namespace {

constexpr int kThreads = kRowThreads;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.44269504088896340736f;
// LDS keys per wave for candidate lists. Ranking reads a list 8 keys at a
// time, so the 8 places after a list hold end markers (INT64_MIN), and a
// list holds at most kCandCap keys.
constexpr int kCandKeys = 256;
constexpr int kListPad = 8;
constexpr int kCandCap = kCandKeys - kListPad;
constexpr uint64_t kSignBit = 0x8000000000000000ull;
// From this K on the chunk threshold uses the lanes' two largest values.
constexpr int kTwoPerLaneFrom = 33;

typedef long long i64x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Records: header {m | e, S | e}, then K keys as {high | e, low | e}.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t record_bytes(int K) { return 16u * (uint32_t)(K + 1); }

__device__ __forceinline__ Rsrc records_rsrc(const TopKParams &p, int64_t pos) {
  const uint32_t rb = record_bytes(p.K);
  return make_rsrc(reinterpret_cast<const char *>(p.records) + pos * p.C * (int64_t)rb,
                   (uint32_t)p.C * rb);
}

__device__ __forceinline__ u32x4 key_words(int64_t k, uint32_t e) {
  const uint64_t u = (uint64_t)k;
  return u32x4{(uint32_t)(u >> 32), e, (uint32_t)u, e};
}
__device__ __forceinline__ uint64_t words_ukey(const u32x4 &w) {
  // the key in unsigned order (sign bit flipped): INT64_MIN, "no key", is 0
  return (((uint64_t)w[0] << 32) | (uint64_t)w[2]) ^ kSignBit;
}
__device__ __forceinline__ bool words_ready(const u32x4 &w, uint32_t e) {
  return ((w[1] == e) & (w[3] == e)) != 0;
}

__device__ __forceinline__ u32x4 load_words(const Rsrc &r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevScope);
}

// Re-polls a pair of tagged words that did not yet show this call's epoch.
__device__ __forceinline__ u32x4 poll_words(Rsrc r, uint32_t off, uint32_t epoch, uint32_t *err_flag) {
  u32x4 w;
  uint32_t spins = 0;
  do {
    __builtin_amdgcn_s_sleep(1);
    w = load_words(r, off);
  } while (!words_ready(w, epoch) && ++spins <= kSpinLimit && !call_failed(err_flag, epoch));
  if (!words_ready(w, epoch)) give_up(err_flag, epoch);
  return w;
}

// ---------------------------------------------------------------------------
// Wave-wide helpers.
// ---------------------------------------------------------------------------
// The k-th largest (1 <= k <= 64) over the lanes of u, in unsigned order.
// Bits are fixed from the top: a bit is set when at least k lanes are at or
// above the prefix with that bit set.
template <class U>
__device__ __forceinline__ U wave_kth_largest(U u, int k) {
  U res = 0;
#pragma unroll
  for (int b = 8 * (int)sizeof(U) - 1; b >= 0; --b) {
    const U c = res | ((U)1 << b);
    res = (__popcll(__ballot(u >= c)) >= k) ? c : res;
  }
  return res;
}

// The same over two values per lane (1 <= k <= 128).
__device__ __forceinline__ uint32_t wave_kth_largest2(uint32_t u, uint32_t w, int k) {
  uint32_t res = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = res | (1u << b);
    res = (__popcll(__ballot(u >= c)) + __popcll(__ballot(w >= c)) >= k) ? c : res;
  }
  return res;
}


// Ranks of the keys of an LDS list of n <= 64 NX keys (distinct, except for
// INT64_MIN): key[x] = list[lane + 64 x], rank[x] = the number of list keys
// above it (INT_MAX past the list end). list[n .. n + 8) must hold INT64_MIN
// (the list is read 8 keys per wait).
template <int NX>
__device__ __forceinline__ void rank_keys(const int64_t *list, int n, int64_t (&key)[4],
                                          int (&rank)[4]) {
  const int lane = lane_here();
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int idx = lane + x * kWave;
    key[x] = idx < n ? list[idx] : INT64_MIN;
    rank[x] = 0;
  }
  for (int j = 0; j < n; j += kListPad) {
    const i64x2 *l2 = reinterpret_cast<const i64x2 *>(list + j);
    const i64x2 a = l2[0], b = l2[1], c = l2[2], d = l2[3];
#pragma unroll
    for (int x = 0; x < NX; ++x)
      rank[x] += (int)(a[0] > key[x]) + (int)(a[1] > key[x]) + (int)(b[0] > key[x]) +
                 (int)(b[1] > key[x]) + (int)(c[0] > key[x]) + (int)(c[1] > key[x]) +
                 (int)(d[0] > key[x]) + (int)(d[1] > key[x]);
  }
#pragma unroll
  for (int x = 0; x < NX; ++x)
    if (lane + x * kWave >= n) rank[x] = INT_MAX;
#pragma unroll
  for (int x = NX; x < 4; ++x) {
    key[x] = INT64_MIN;
    rank[x] = INT_MAX;
  }
}

__device__ __forceinline__ void rank_list(const int64_t *list, int n, int64_t (&key)[4],
                                          int (&rank)[4]) {
  if (n <= kWave) rank_keys<1>(list, n, key, rank);
  else if (n <= 2 * kWave) rank_keys<2>(list, n, key, rank);
  else if (n <= 3 * kWave) rank_keys<3>(list, n, key, rank);
  else rank_keys<4>(list, n, key, rank);
}

// ---------------------------------------------------------------------------
// Reduction of one chunk to its record. On return lanes hold (key[x],
// rank[x]) pairs: the keys of rank < K are the chunk's top-K (INT64_MIN
// where the chunk has fewer than K columns); mw and S are the header.
// ---------------------------------------------------------------------------
struct ChunkTop {
  int64_t key[4];
  int rank[4];
  float mw;
  float S;
};

template <bool VEC>
__device__ __forceinline__ void reduce_chunk_topk(const TopKParams &p, int64_t row, float T,
                                                  int32_t chunk, float4 (&v)[kQ], int64_t *cand,
                                                  ChunkTop &out) {
  const int lane = lane_id();
  const int32_t V = p.vocab;
  const int K = p.K;
  const float tc = clamp_temp(T);
  const Recip rc = recip_of_uniform(tc);
  const double rtc = rc.hi;
  const int32_t c0 = chunk * kChunkCols;
  // column of element 0 of this lane. The columns are the same for every
  // row of this wave: without this the compiler computes the fallback's
  // keys of all 32 columns once, outside the row loop, and spills them.
  int32_t cl = c0 + 4 * lane;
  __asm__ volatile("" : "+v"(cl));
  auto col_of = [&](uint32_t k) -> int32_t {
    return cl + 4 * (int32_t)(k >> 2) * kWave + (int32_t)(k & 3u);
  };

  // ---- mask the row end, scale s = fl32(x / Tc) ----
  const int32_t left = V - c0;
  if (left < kChunkCols) {
    // columns left from this lane's first one; the lane number is taken
    // afresh here, else the compiler keeps the 32 comparisons across the
    // row loop as scalar register pairs (and spills them)
    const int32_t lim = left - 4 * lane_here();
#pragma unroll
    for (int j = 0; j < kQ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        set_comp(v[j], i, (4 * j * kWave + i < lim) ? comp(v[j], i) : -INFINITY);
  }
  float mt = -INFINITY;
  if (T == 1.0f) {  // x / 1 = x
#pragma unroll
    for (int j = 0; j < kQ; ++j) mt = fmaxf(mt, max4(v[j]));
  } else {
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      v[j].x = scale(v[j].x, rtc);
      v[j].y = scale(v[j].y, rtc);
      v[j].z = scale(v[j].z, rtc);
      v[j].w = scale(v[j].w, rtc);
      mt = fmaxf(mt, max4(v[j]));
    }
  }
  const float mw = wave_max_f32(mt);

  // ---- S = sum exp(s - m) of the chunk (1 <= S <= 2048 unless empty) ----
  const float mu = (mw == -INFINITY) ? 0.0f : mw;
  float St = 0.0f;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) St += __builtin_amdgcn_exp2f((comp(v[j], i) - mu) * kLog2e);
  out.mw = mw;
  out.S = wave_allreduce(St, SumF());  // the record header holds it as fp32
  // (after the sum, which a change of one subnormal unit in s cannot alter;
  // the order of the values below, the keys, needs them exact)
  // From Tc = 2 on, a quotient below 2^-126 can be a midpoint of the
  // subnormal grid that the product form rounds the wrong way by one unit
  // (device_common.h): such results are recomputed exactly from their raw
  // logits. Rare (values within 2^-126 T of zero).
  if (tc >= 2.0f) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < 4 * kQ; ++k) any |= fabsf(comp(v[k >> 2], k & 3)) <= 0x1p-126f;
    if (__ballot(any) != 0) {
#pragma unroll
      for (int k = 0; k < 4 * kQ; ++k) {
        if (fabsf(comp(v[k >> 2], k & 3)) <= 0x1p-126f) {
          const float x = p.logits[row * p.ld + col_of((uint32_t)k)];
          set_comp(v[k >> 2], k & 3, scale_dd(x, rc));
        }
      }
      mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < kQ; ++j) mt = fmaxf(mt, max4(v[j]));
      // the header's maximum must equal the largest key's value
      out.mw = wave_max_f32(mt);
    }
  }

  // ---- threshold: the K-th largest lane maximum (or of the lanes' two
  // largest values) ----
  uint32_t uk;
  if (K < kTwoPerLaneFrom) {
    uk = wave_kth_largest<uint32_t>((uint32_t)key32(mt) ^ 0x80000000u, K);
  } else {
    float a = -INFINITY, b = -INFINITY;  // the lane's largest and second largest
#pragma unroll
    for (int k = 0; k < 4 * kQ; ++k) {
      const float x = comp(v[k >> 2], k & 3);
      b = __builtin_amdgcn_fmed3f(a, b, x);
      a = fmaxf(a, x);
    }
    uk = wave_kth_largest2((uint32_t)key32(a) ^ 0x80000000u, (uint32_t)key32(b) ^ 0x80000000u, K);
  }
  const float vk = key32_value((int32_t)(uk ^ 0x80000000u));
  // Bit 31 - k of cm: element k is a candidate (s >= v_K). With v_K > -inf
  // the K lanes whose maxima reach v_K give at least K candidates, all real
  // columns (masked ones are -inf).
  uint32_t cm = 0;
#pragma unroll
  for (int j = 0; j < kQ; ++j) cm = push4_bits_ge(cm, v[j].x, v[j].y, v[j].z, v[j].w, vk, vk, vk, vk);
  int total;
  const int off = wave_prefix(__popc(cm), total);

  if (vk != -INFINITY && total <= kCandCap) {
    int o = off;
    for (uint32_t c2 = cm; c2 != 0;) {
      const uint32_t k = (uint32_t)__builtin_clz(c2);
      c2 &= ~(0x80000000u >> k);
      cand[o++] = key64(element_at(v, k), col_of(k));
    }
    if (lane < kListPad) cand[total + lane] = INT64_MIN;
    wave_lds_order();
    rank_list(cand, total, out.key, out.rank);
    wave_lds_order();
  } else {
    // exact fallback: K rounds of "largest key below the previous one";
    // lane k keeps the key of rank k
    int64_t prev = INT64_MAX, mine = INT64_MIN;
    for (int r = 0; r < K; ++r) {
      int64_t best = INT64_MIN;
#pragma unroll
      for (int k = 0; k < 4 * kQ; ++k) {
        const int32_t c = col_of((uint32_t)k);
        const int64_t key = (c < V) ? key64(comp(v[k >> 2], k & 3), c) : INT64_MIN;
        best = (key < prev && key > best) ? key : best;
      }
      best = wave_allreduce(best, MaxI64());
      if (lane == r) mine = best;
      prev = best;
    }
    out.key[0] = mine;
    out.rank[0] = lane;
#pragma unroll
    for (int x = 1; x < 4; ++x) {
      out.key[x] = INT64_MIN;
      out.rank[x] = INT_MAX;
    }
  }
}

__device__ __forceinline__ void publish_record(const TopKParams &p, int64_t pos, int32_t chunk,
                                               const ChunkTop &t) {
  const Rsrc r = records_rsrc(p, pos);
  const uint32_t base = (uint32_t)chunk * record_bytes(p.K);
#pragma unroll
  for (int x = 0; x < 4; ++x)
    if (t.rank[x] < p.K)
      __builtin_amdgcn_raw_buffer_store_b128(key_words(t.key[x], p.epoch), r,
                                             base + 16u * (uint32_t)(t.rank[x] + 1), 0, kDevScope);
  if (lane_id() == 0) {
    const u32x4 h = {__float_as_uint(t.mw), p.epoch, __float_as_uint(t.S), p.epoch};
    __builtin_amdgcn_raw_buffer_store_b128(h, r, base, 0, kDevScope);
  }
}

__device__ __forceinline__ int64_t load_uniform_i64(const int64_t *p) {
  return *(const __attribute__((address_space(4))) int64_t *)p;
}
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t *p) {
  return *(const __attribute__((address_space(4))) int32_t *)p;
}

// Columns of the row whose scaled value reaches M (its maximum): one pass
// over the row by the merger, for rows whose K largest keys all tie at M.
__device__ __forceinline__ int count_at_max(const TopKParams &p, int64_t row, float T, float M) {
  const float tc = clamp_temp(T);
  const Recip rc = recip_of(tc);
  const float *x = p.logits + row * p.ld;
  int cnt = 0;
  for (int32_t c = lane_here(); c < p.vocab; c += kWave) cnt += scale_any(x[c], rc, tc) >= M ? 1 : 0;
  return wave_allreduce(cnt, SumI());
}

// One stash row: column 0 holds the argmax; after it come the request's
// own token ids or else its K_out largest keys; the cells left up to the
// width hold token 0 at -inf; and the argmax's rank
// (the columns at or above its value). buf holds the row's K largest keys
// in rank order, M its maximum and logS = log sum exp(s - M).
__device__ __forceinline__ void write_stash_row(const TopKParams &p, int64_t pos, int64_t row,
                                             const int64_t *buf, float M, double logS) {
  const int lane = lane_here();
  const int K = p.K;
  const float T = load_uniform(p.kept_temp + pos);
  const int64_t dst = load_uniform_i64(LATE_ARG(TopKParams, kept_dst) + pos);
  const int32_t j = load_uniform_i32(LATE_ARG(TopKParams, kept_req) + pos);
  const int32_t W = LATE_ARG(TopKParams, width);
  const bool logits_mode = LATE_ARG(TopKParams, logits_mode) != 0;
  int32_t *oid = LATE_ARG(TopKParams, out_ids32) + dst * W;
  float *olp = LATE_ARG(TopKParams, out_lp) + dst * W;
  auto value = [&](float s) -> float {
    return logits_mode ? s : (float)(((double)s - (double)M) - logS);
  };
  // ties at the maximum among the K keys; when all K tie, count the row
  const int64_t mine = lane < K ? buf[lane] : INT64_MIN;
  int ties = __popcll(__ballot(lane < K && (int32_t)(mine >> 32) == key32(M)));
  if (ties == K) ties = count_at_max(p, row, T, M);
  int n = LATE_ARG(TopKParams, K_out);
  bool by_ids = false;
  const int32_t *ids = LATE_ARG(TopKParams, ids);
  const int64_t ids_stride = LATE_ARG(TopKParams, ids_stride);
  if (ids != nullptr) {
    const int32_t c = load_uniform_i32(LATE_ARG(TopKParams, num_ids) + j);
    if (c > 0) {
      by_ids = true;
      n = (int)min((int64_t)min(c, W - 1), ids_stride);
    }
  }
  if (lane == 0) {
    oid[0] = key64_col(buf[0]);
    olp[0] = value(key32_value((int32_t)(buf[0] >> 32)));
    LATE_ARG(TopKParams, out_ranks)[dst] = ties;
  }
  if (by_ids) {
    const float tc = clamp_temp(T);
    const Recip rc = recip_of(tc);
    const int32_t *idr = ids + (int64_t)j * ids_stride;
    for (int i = lane; i < n; i += kWave) {
      const int32_t id = idr[i];
      float v = -INFINITY;
      if (id >= 0 && id < p.vocab) v = value(scale_any(p.logits[row * p.ld + id], rc, tc));
      else atomicOr(p.err_flag, kErrIndex);
      oid[1 + i] = id;
      olp[1 + i] = v;
    }
  } else if (lane < n) {
    oid[1 + lane] = key64_col(mine);
    olp[1 + lane] = value(key32_value((int32_t)(mine >> 32)));
  }
  for (int c = 1 + n + lane; c < W; c += kWave) {
    oid[c] = 0;
    olp[c] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// The merger's work for the kept row at position pos (row index `row`).
// buf is the wave's LDS list area: the running top-K in [0, K), the keys
// waiting to be ranked in [K, K + nb).
// ---------------------------------------------------------------------------
__device__ void merge_row_topk(const TopKParams &p, int64_t pos, int64_t row, int64_t *buf) {
  const int lane = lane_here();
  const int K = p.K, C = p.C;
  const uint32_t rb = record_bytes(K);
  const Rsrc r = records_rsrc(p, pos);

  // ---- headers, chunk maxima and second keys ----
  // Records q = lane + 64 i. Their header and first two keys are read at
  // once; the keys of records 0 and 1 of the lane stay in registers, since
  // on typical rows few keys past the second of a record reach the bound.
  float ml = -INFINITY;
  double Sl = 0.0;
  uint64_t umax = 0;  // largest chunk maximum of the lane, unsigned order
  auto add_header = [&](const u32x4 &h) {
    const float mq = __uint_as_float(h[0]);
    const float Sq = __uint_as_float(h[2]);
    if (Sq > 0.0f) {
      if (mq > ml) {
        Sl = Sl * (double)__builtin_amdgcn_exp2f((ml - mq) * kLog2e) + (double)Sq;
        ml = mq;
      } else {
        Sl += (double)Sq * (double)__builtin_amdgcn_exp2f((mq - ml) * kLog2e);
      }
    }
  };
  auto ready = [&](u32x4 w, uint32_t off) {
    return words_ready(w, p.epoch) ? w : poll_words(r, off, p.epoch, p.err_flag);
  };
  const u32x4 none = {0u, 0u, 0u, 0u};
  const bool has0 = lane < C, has1 = lane + kWave < C, two = K > 1;
  const uint32_t o0 = (uint32_t)lane * rb, o1 = (uint32_t)(lane + kWave) * rb;
  u32x4 h0 = none, w00 = none, w01 = none, h1 = none, w10 = none, w11 = none;
  if (has0) {
    h0 = load_words(r, o0);
    w00 = load_words(r, o0 + 16u);
    if (two) w01 = load_words(r, o0 + 32u);
  }
  if (has1) {
    h1 = load_words(r, o1);
    w10 = load_words(r, o1 + 16u);
    if (two) w11 = load_words(r, o1 + 32u);
  }
  if (has0) {
    h0 = ready(h0, o0);
    w00 = ready(w00, o0 + 16u);
    if (two) w01 = ready(w01, o0 + 32u);
    add_header(h0);
    umax = words_ukey(w00);
  }
  if (has1) {
    h1 = ready(h1, o1);
    w10 = ready(w10, o1 + 16u);
    if (two) w11 = ready(w11, o1 + 32u);
    add_header(h1);
    umax = max(umax, words_ukey(w10));
  }
  for (int q = lane + 2 * kWave; q < C; q += kWave) {
    const uint32_t o = (uint32_t)q * rb;
    u32x4 h = load_words(r, o), w0 = load_words(r, o + 16u);
    add_header(ready(h, o));
    umax = max(umax, words_ukey(ready(w0, o + 16u)));
  }
  const float M = wave_max_f32(ml);
  const double S = wave_allreduce(
      Sl > 0.0 ? Sl * (double)__builtin_amdgcn_exp2f((ml - M) * kLog2e) : 0.0, SumD());
  const double logS = log_d(S);  // log Z = M + logS

  // ---- lower bound of the row's K-th key ----
  // With at least K lanes holding records, the K-th largest of the lanes'
  // maxima is one (K distinct keys reach it), and so is that key with its
  // low word cleared, whose high word is the K-th largest high word.
  // Otherwise every key is read.
  uint64_t t = 1;  // unsigned order; 0 is "no key"
  if (min(C, kWave) >= K)
    t = max((uint64_t)wave_kth_largest<uint32_t>((uint32_t)(umax >> 32), K) << 32, (uint64_t)1);

  // ---- keys at or above t, ranked with the running top-K ----
  if (lane < K) buf[lane] = INT64_MIN;
  int nb = 0;
  const int B = kCandCap - K;
  auto flush = [&]() {
    const int n = K + nb;
    if (lane < kListPad) buf[n + lane] = INT64_MIN;
    wave_lds_order();
    int64_t key[4];
    int rank[4];
    rank_list(buf, n, key, rank);
    wave_lds_order();
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (rank[x] < K) buf[rank[x]] = key[x];
    wave_lds_order();
    nb = 0;
    // keys below the current K-th can no longer enter
    const int64_t kth = buf[K - 1];
    t = max(t, (uint64_t)kth ^ kSignBit);
  };
  // Appends the keys kk[x] with bit x of fl set, ranking whenever the list
  // is full.
  auto append = [&](const int64_t (&kk)[4], uint32_t fl) {
    int total;
    const int off = wave_prefix(__popc(fl), total);
    for (int done = 0; done < total;) {
      if (nb == B) flush();
      const int room = B - nb;
      int o = off;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if ((fl >> x) & 1) {
          const int g = o - done;
          if (g >= 0 && g < room) buf[K + nb + g] = kk[x];
          ++o;
        }
      }
      const int took = min(room, total - done);
      nb += took;
      done += took;
    }
  };
  // the first two keys of records 0 and 1 of the lane
  uint64_t later = 0;  // records 0 and 1 still to be read from slot 2 on
  {
    const uint64_t u[4] = {words_ukey(w00), words_ukey(w01), words_ukey(w10), words_ukey(w11)};
    const bool in[4] = {has0, has0 && two, has1, has1 && two};
    int64_t kk[4];
    uint32_t fl = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      kk[x] = (int64_t)(u[x] ^ kSignBit);
      if (in[x] && u[x] >= t) fl |= 1u << x;
    }
    if (K > 2) later = (uint64_t)((fl >> 1) & 1) | ((uint64_t)((fl >> 3) & 1) << 1);
    append(kk, fl);
  }
  // the other records from slot 0, records 0 and 1 from slot 2, each while
  // its keys reach t (a record is sorted)
  const int nq = lane < C ? (C - 1 - lane) / kWave + 1 : 0;  // records of this lane
  const int nqmax = (C + kWave - 1) / kWave;
  uint64_t act = nq > 2 ? (nq >= 64 ? ~0ull : (1ull << nq) - 1ull) & ~3ull : 0ull;
  for (int s = 0; s < K; ++s) {
    if (s == 2) {
      act |= later;
      later = 0;
    }
    if (__ballot((act | later) != 0) == 0) break;
    if (__ballot(act != 0) == 0) continue;
    const uint32_t soff = 16u * (uint32_t)(s + 1);
    for (int q0 = 0; q0 < nqmax; q0 += 4) {
      u32x4 w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t q = (uint32_t)(lane + (q0 + x) * kWave);
        w[x] = ((act >> (q0 + x)) & 1) ? load_words(r, q * rb + soff) : none;
      }
      int64_t kk[4];
      uint32_t fl = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kk[x] = INT64_MIN;
        if ((act >> (q0 + x)) & 1) {
          const uint32_t q = (uint32_t)(lane + (q0 + x) * kWave);
          const uint64_t u = words_ukey(ready(w[x], q * rb + soff));
          if (u >= t) {
            kk[x] = (int64_t)(u ^ kSignBit);
            fl |= 1u << x;
          } else {
            act &= ~(1ull << (q0 + x));
          }
        }
      }
      append(kk, fl);
    }
    if (s + 1 == K) act = 0;
  }
  flush();

  if (p.stash) {
    write_stash_row(p, pos, row, buf, M, logS);
  } else if (lane < K) {
    const int64_t key = buf[lane];
    const float s = key32_value((int32_t)(key >> 32));
    p.out_idx[row * K + lane] = key64_col(key);
    p.out_vals[row * K + lane] = (float)(((double)s - (double)M) - logS);
  }
  wave_lds_order();
  if (lane == 0) store_row_result(p.rowres, pos, __float_as_uint(M), 0u, p.epoch);
}

// ---------------------------------------------------------------------------
// The kernel. Global wave gw belongs to group gw / C as member gw % C: the
// group reduces one kept row at a time (positions from a RowDealer), the
// member chunk `member` of each. The merger of the group's n-th row is
// member n % C; it merges row n after reducing row n + kMergeLag. Before merging,
// every member waits for the row result of row n - kPaceLag, which keeps
// the waves of a SIMD in step. A merge delays its merger's next chunks;
// the merger of a later row waits for such a late chunk only when the
// delay exceeds kMergeLag chunk periods.
// ---------------------------------------------------------------------------
constexpr int kMergeLag = 2;
constexpr int kPaceLag = kMergeLag + 2;

template <bool VEC>
__global__ __launch_bounds__(kThreads, 4) void topk_kernel(TopKParams p) {
  __shared__ float4 stage[VEC ? kWaves * kChunkQuads : 1];
  __shared__ __attribute__((aligned(16))) int64_t lists[kWaves * kCandKeys];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int gw = (int)blockIdx.x * kWaves + wave;
  const int group = gw / p.C;
  const int member = gw - group * p.C;
  if (group >= p.n_groups) return;
  const int64_t n_kept = load_uniform_i64(p.kept + p.rows);
  if (group >= n_kept) return;
  const int32_t chunk = member;
  const int64_t G = p.n_groups;
  const bool leader = member == 0;
  RowDealer d;
  d.ring = p.rings + (int64_t)group * (kRingBytes / 8);
  d.counter = p.counters + (p.epoch & 1);
  d.limit = n_kept;
  d.first = kDealAhead * G;
  d.group = group;
  d.G = G;
  d.epoch = p.epoch;
  auto row_at = [&](int64_t pos) -> int64_t { return load_uniform_i64(p.kept + (pos >= 0 ? pos : 0)); };
  float4 *const buf = stage + (VEC ? wave * kChunkQuads : 0);
  int64_t *const list = lists + wave * kCandKeys;
  // as in the row-statistics kernel, the copy past the last row still
  // issues (through a zero-size descriptor) so that every path issues the
  // same operations
  const uint32_t bytes = chunk_bytes(chunk * kChunkCols, p.vocab);
  auto copy_chunk = [&](int64_t pos, int64_t row) {
    chunk_copy_bytes(buf, pos >= 0 ? p.logits + row * p.ld + chunk * kChunkCols : p.logits,
                     pos >= 0 ? bytes : 0u);
  };

  // positions of iterations n (pos), n + 1 and n - 1 .. n - kPaceLag (hist)
  int64_t pos = group, pos_next = d.static_pos(1);
  int64_t row = row_at(pos), row_next = row_at(pos_next);
  int64_t hist[kPaceLag];
#pragma unroll
  for (int i = 0; i < kPaceLag; ++i) hist[i] = -1;
  bool claiming = leader;
  int mturn = 0;  // (n - kMergeLag) % C
  if constexpr (VEC) copy_chunk(pos, row);
  for (int n = 0; pos >= 0; ++n) {
    const int64_t pace_pos = hist[kPaceLag - 1];
    u32x4 rr = load_row_result(p.rowres, pace_pos >= 0 ? pace_pos : pos);
    u32x4 slot = d.load_slot(n + 2);
    uint32_t claim = 0;
    if (claiming) claim = d.claim();
    compiler_fence();
    float4 cur[kQ];
    if constexpr (VEC) {
      // after this row's copy came, in the previous row, at least its record
      // header store, then this row's row-result and slot loads and (member
      // 0) its claim
      if (leader) wait_vm<3>();
      else wait_vm<2>();
      lds_read_chunk(cur, buf);
      compiler_fence();
      copy_chunk(pos_next, row_next);
      compiler_fence();
    } else {
      chunk_load(cur, p.logits + row * p.ld, chunk * kChunkCols, p.vocab);
    }
    ChunkTop t;
    reduce_chunk_topk<VEC>(p, row, load_uniform(p.kept_temp + pos), chunk, cur, list, t);
    // consume the loads issued before the copy here, before the record
    // stores, so that their wait does not wait for the copy above
    __asm__ volatile("" ::"v"(rr), "v"(slot), "v"(claim));
    compiler_fence();
    const int64_t pos_after = n + 2 < kDealAhead ? d.static_pos(n + 2) : d.slot_pos(slot, n + 2, p.err_flag);
    const int64_t row_after = row_at(pos_after);
    if (leader) {
      int64_t q = -1;
      if (claiming) {
        q = d.claimed_pos(claim);
        claiming = q >= 0;
      }
      d.post(n + kDealAhead, q);
    }
    publish_record(p, pos, chunk, t);
    compiler_fence();
    if (pace_pos >= 0) rr = wait_row_result(p.rowres, pace_pos, rr, p.epoch, p.err_flag);
    if (n >= kMergeLag) {
      if (mturn == member) {
        const int64_t mpos = hist[kMergeLag - 1];
        merge_row_topk(p, mpos, row_at(mpos), list);
      }
      if (++mturn == p.C) mturn = 0;
    }
#pragma unroll
    for (int i = kPaceLag - 1; i > 0; --i) hist[i] = hist[i - 1];
    hist[0] = pos;
    pos = pos_next;
    pos_next = pos_after;
    row = row_next;
    row_next = row_after;
  }
  // the last kMergeLag rows (fewer if the group has fewer rows)
#pragma unroll
  for (int i = kMergeLag - 1; i >= 0; --i) {
    if (hist[i] < 0) continue;
    if (mturn == member) merge_row_topk(p, hist[i], row_at(hist[i]), list);
    if (++mturn == p.C) mturn = 0;
  }
}

// ---------------------------------------------------------------------------
// Kept-row list: kept[0 .. n) = the rows of kept slots in order, kept[rows]
// = n, and kept_temp[i] = the temperature of row kept[i]; also zeroes the
// row-claim counters. One workgroup; thread t handles a contiguous range of
// rows.
// ---------------------------------------------------------------------------
constexpr int kListThreads = 1024;

__global__ __launch_bounds__(kListThreads) void kept_rows_kernel(const uint8_t *keep,
                                                               const float *temps, int64_t rows,
                                                               int64_t canvas_len, int64_t *kept,
                                                               float *kept_temp,
                                                               uint32_t *counters) {
  __shared__ int64_t wave_tot[kListThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t per = (rows + kListThreads - 1) / kListThreads;
  const int64_t r0 = min(rows, (int64_t)tid * per), r1 = min(rows, r0 + per);
  int64_t cnt = 0;
  for (int64_t r = r0; r < r1;) {
    const int64_t slot = r / canvas_len;
    const int64_t end = min(r1, (slot + 1) * canvas_len);
    if (keep[slot]) cnt += end - r;
    r = end;
  }
  // exclusive prefix over the workgroup
  int64_t incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t o = __shfl_up(incl, (unsigned)d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int64_t off = incl - cnt;
  for (int w = 0; w < wave; ++w) off += wave_tot[w];
  for (int64_t r = r0; r < r1;) {
    const int64_t slot = r / canvas_len;
    const int64_t end = min(r1, (slot + 1) * canvas_len);
    if (keep[slot]) {
      const float T = temps[slot];
      for (; r < end; ++r) {
        kept_temp[off] = T;
        kept[off++] = r;
      }
    }
    r = end;
  }
  if (tid == kListThreads - 1) {
    kept[rows] = off;
    // row-claim counters of the kernel that follows and of the next call
    counters[0] = 0u;
    counters[1] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Kept-row list of the stash: each kept request j, in order, contributes
// the rows src[j] * canvas_len + q for q < min(valid[j], canvas_len), with
// kept_temp = temps[j], kept_dst = slots[j] * positions + q and kept_req = j;
// kept[rows] = the count. A kept request whose rows fall outside the logits
// or whose slot falls outside the stash is skipped and flags kErrIndex.
// Also zeroes the row-claim counters. One workgroup; thread t handles a
// contiguous range of requests.
// ---------------------------------------------------------------------------
constexpr int kStashLdsRequests = 4096;  // requests whose offsets fit in LDS

__global__ __launch_bounds__(kListThreads) void stash_rows_kernel(TopKParams p) {
  __shared__ int64_t wave_tot[kListThreads / kWave];
  __shared__ int64_t req_off[kStashLdsRequests + 1];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t per = (p.m + kListThreads - 1) / kListThreads;
  const int64_t j0 = min(p.m, (int64_t)tid * per), j1 = min(p.m, j0 + per);
  // rows of request j; -1 for a kept request with an index out of range
  auto rows_of = [&](int64_t j) -> int64_t {
    if (!p.keep[j]) return 0;
    const int64_t n = min((int64_t)max(p.valid[j], 0), p.canvas_len);
    if (n == 0) return 0;
    const int64_t src = p.src[j], slot = p.slots[j];
    if (src < 0 || src * p.canvas_len + n > p.logits_rows || slot < 0 || slot >= p.stash_slots)
      return -1;
    return n;
  };
  int64_t cnt = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const int64_t n = rows_of(j);
    if (n > 0) cnt += n;
    else if (n < 0) atomicOr(p.err_flag, kErrIndex);
  }
  // exclusive prefix over the workgroup
  int64_t incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t o = __shfl_up(incl, (unsigned)d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int64_t off = incl - cnt;
  for (int w = 0; w < wave; ++w) off += wave_tot[w];
  int64_t total = 0;
  for (int w = 0; w < kListThreads / kWave; ++w) total += wave_tot[w];
  auto put = [&](int64_t i, int64_t j, int64_t q) {
    p.kept[i] = (int64_t)p.src[j] * p.canvas_len + q;
    p.kept_temp[i] = p.temps[j];
    p.kept_dst[i] = (int64_t)p.slots[j] * p.positions + q;
    p.kept_req[i] = (int32_t)j;
  };
  if (p.m <= kStashLdsRequests) {
    // every thread writes consecutive entries: the request of entry i is
    // the last one whose first entry is at or below i
    for (int64_t j = j0; j < j1; ++j) {
      req_off[j] = off;
      off += max(rows_of(j), (int64_t)0);
    }
    if (tid == 0) req_off[p.m] = total;
    __syncthreads();
    for (int64_t i = tid; i < total; i += kListThreads) {
      int64_t lo = 0, hi = p.m;  // req_off[lo] <= i < req_off[hi]
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (req_off[mid] <= i) lo = mid;
        else hi = mid;
      }
      put(i, lo, i - req_off[lo]);
    }
  } else {
    for (int64_t j = j0; j < j1; ++j) {
      const int64_t n = rows_of(j);
      for (int64_t q = 0; q < n; ++q, ++off) put(off, j, q);
    }
  }
  if (tid == kListThreads - 1) {
    p.kept[p.rows] = total;
    p.counters[0] = 0u;
    p.counters[1] = 0u;
  }
}

}  // namespace

static const void *topk_kernel_ptr(bool vec) {
  return vec ? reinterpret_cast<const void *>(&topk_kernel<true>)
             : reinterpret_cast<const void *>(&topk_kernel<false>);
}

hipError_t topk_resident_blocks(bool vec, int *blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, topk_kernel_ptr(vec), kThreads,
                                                      0);
}

hipError_t kept_rows_launch(const TopKParams &p, hipStream_t stream) {
  kept_rows_kernel<<<dim3(1), dim3(kListThreads), 0, stream>>>(p.keep, p.temps, p.rows,
                                                                p.canvas_len, p.kept, p.kept_temp,
                                                                p.counters);
  return hipGetLastError();
}

hipError_t stash_rows_launch(const TopKParams &p, hipStream_t stream) {
  stash_rows_kernel<<<dim3(1), dim3(kListThreads), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t topk_launch(const TopKParams &p, int grid, hipStream_t stream) {
  if (p.stash)
    stash_rows_kernel<<<dim3(1), dim3(kListThreads), 0, stream>>>(p);
  else
    kept_rows_kernel<<<dim3(1), dim3(kListThreads), 0, stream>>>(
        p.keep, p.temps, p.rows, p.canvas_len, p.kept, p.kept_temp, p.counters);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TopKParams arg = p;
  void *args[] = {&arg};
  return hipLaunchCooperativeKernel(topk_kernel_ptr(p.vec_ok != 0), dim3(grid), dim3(kThreads), args,
                                    0, stream);
}

}  // namespace rowstats
