// One-pass row statistics (argmax, Gumbel-max sample, entropy, optional
// softmax) of temperature-scaled fp32 logits on gfx950.
//
// Method: vLLM API page "diffusion_gemma_sampler", module docstring (a
// single read of each row keeps a running maximum and sum, generates the
// noise in place and stores the probabilities a single time) and sample_row_stats /
// sample_row_stats_reference (the statistics and the greedy rule).
//
// Work split. A row is cut into C chunks of 2048 columns, and a group of C
// member waves reduces one row at a time, one chunk each; each group walks
// its own rows. A wave keeps its chunk in registers (8 float4 per lane), so
// each logit is read from HBM once, and waves never meet at a barrier.
// While a wave reduces one chunk, its next chunk is copied from HBM into
// the wave's LDS buffer (buffer_load ... lds).
//
// A wave reduces its chunk to a summary relative to its own maximum m:
//   (m, lowest column of m, S = sum 2^32 exp(s - m),
//    W = sum 2^32 exp(s - m) (s - m), best perturbed score z, its column)
// and stores it in global scratch as eight 64-bit words, each carrying the
// call's epoch in its high half; stores and loads of these words are
// device-scope coherent and 64-bit words are never torn, so a word that
// shows the current epoch is final. One member per row (the merger,
// rotating over the members) polls the row's summaries one or two chunks
// later (kMergeLag), merges them, writes the row's argmax, sample and
// entropy, and publishes (m, 1 / S) of the row. Every member waits for that
// row result two chunks after the merge (kLag): with probs it then writes
// its chunk's probabilities from the exp values it kept in registers, so
// the exchange overlaps chunks of work. The launch is cooperative (every
// wave resident), so each wait ends.
//
// Gumbel sample (T > 0). The wave's argmax a gives a lower bound
// zlb = s_a + g_a on its best perturbed score. A column can reach zlb only
// if s >= zlb - 22.8739 (the largest Gumbel value a 32-bit word yields), so
// quads below that skip the Philox draw; a drawn column can reach zlb only
// if 1 - u <= exp(s - zlb), which follows from -log u >= 1 - u and reuses
// the column's exp value (tested per quad first, then per column). The few
// columns passing get an fp32 score estimate; those within 2^-8 of the best
// are scored exactly in fp64, and the best score wins (ties to the lower
// column).
#include "chunk_common.h"
#include "device_common.h"
#include "device_math.h"
#include "rowstats_internal.h"

#include <float.h>
#include <limits.h>

namespace rowstats {

constexpr int kThreads = kRowThreads;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.44269504088896340736f;
// 2^32 exp(-22.8739) = 0.49998, lowered for the 2^-13 error of -log u and
// the rounding of e: a quad whose exp values are all below kQuadSkip / a,
// a = -log u of the bound's word, cannot reach the bound.
constexpr float kQuadSkip = 0.4993f;
constexpr float kTestMargin = 1.0f + 0x1p-10f;

// A wave, chunk or row summary relative to its own maximum m.
struct Tuple {
  float m;
  int32_t am;
  double S;
  double W;
  double zb;  // best perturbed score z = s + g of the summarised columns
  int32_t zc;  // its column
  int32_t zx;  // 1: zb is exact (fp64); 0: fp32 estimate, within 2^-9 of exact
};

__device__ __forceinline__ Tuple empty_tuple() {
  Tuple t;
  t.m = -INFINITY;
  t.am = INT_MAX;
  t.S = 0.0;
  t.W = 0.0;
  t.zb = -INFINITY;
  t.zc = INT_MAX;
  t.zx = 1;
  return t;
}

// Adds summary t, rescaled from its maximum to m, into (S, W). The factors
// exp(t.m - m) are fp32 (relative error near 1e-7); the sums are fp64.
__device__ __forceinline__ void add_rescaled(const Tuple &t, float m, double &S, double &W) {
  if (t.S > 0.0) {
    const float dm = fmaxf(t.m - m, -FLT_MAX);  // <= 0
    const double f = (double)__builtin_amdgcn_exp2f(dm * kLog2e);
    S += t.S * f;
    W += f * (t.W + t.S * (double)dm);
  }
}

// Temperature slot of a row, row / canvas_len, as (row * slot_mul) >> slot_shift
// (exact for every row below 2^31): scalar arithmetic, where a 64-bit
// division would go through vector registers.
__device__ __forceinline__ int64_t slot_of(const RowStatsParams &p, int64_t row) {
  return (int64_t)(((uint64_t)(uint32_t)row * p.slot_mul) >> p.slot_shift);
}

// Merge of two summaries.
__device__ __forceinline__ Tuple combine(const Tuple &a, const Tuple &b) {
  Tuple r;
  r.m = fmaxf(a.m, b.m);
  r.S = 0.0;
  r.W = 0.0;
  add_rescaled(a, r.m, r.S, r.W);
  add_rescaled(b, r.m, r.S, r.W);
  r.am = min(a.m == r.m ? a.am : INT_MAX, b.m == r.m ? b.am : INT_MAX);
  r.zb = fmax(a.zb, b.zb);
  r.zc = min(a.zb == r.zb ? a.zc : INT_MAX, b.zb == r.zb ? b.zc : INT_MAX);
  r.zx = a.zx & b.zx;
  return r;
}

// Merge of the summaries held by the 64 lanes; every lane gets the result.
__device__ __forceinline__ Tuple wave_merge(const Tuple &t) {
  Tuple r;
  r.m = wave_max_f32(t.m);
  double S = 0.0, W = 0.0;
  add_rescaled(t, r.m, S, W);
  r.S = wave_allreduce(S, SumD());
  r.W = wave_allreduce(W, SumD());
  r.am = wave_allreduce(t.m == r.m ? t.am : INT_MAX, MinI());
  r.zb = wave_allreduce(t.zb, MaxD());
  r.zc = wave_allreduce(t.zb == r.zb ? t.zc : INT_MAX, MinI());
  r.zx = wave_allreduce(t.zx, MinI());
  return r;
}

// ---------------------------------------------------------------------------
// Tagged scratch words. A member's summary is eight 64-bit words, payload in
// the low half and the epoch in the high half: m, argmax, S (fp32), W (fp32),
// the two halves of the best score, its column, the score's exactness flag.
// ---------------------------------------------------------------------------
__device__ __forceinline__ Rsrc tuple_rsrc(const RowStatsParams &p, int64_t row) {
  return make_rsrc(p.tuples + row * p.C * (kTupleBytes / 8), (uint32_t)(p.C * kTupleBytes));
}

__device__ __forceinline__ uint32_t tuple_payload(const Tuple &t, int k) {
  switch (k) {
    case 0: return __float_as_uint(t.m);
    case 1: return (uint32_t)t.am;
    case 2: return __float_as_uint((float)t.S);
    case 3: return __float_as_uint((float)t.W);
    case 4: return (uint32_t)(uint64_t)__double_as_longlong(t.zb);
    case 5: return (uint32_t)((uint64_t)__double_as_longlong(t.zb) >> 32);
    case 6: return (uint32_t)t.zc;
    default: return (uint32_t)t.zx;
  }
}

// Lanes 0..3 store two tagged words each (one 16-byte store instruction).
__device__ __forceinline__ void publish_tuple(const Rsrc &r, int member, const Tuple &t,
                                              uint32_t epoch) {
  const int lane = lane_here();
  if (lane < 4) {
    const u32x4 v = {tuple_payload(t, 2 * lane), epoch, tuple_payload(t, 2 * lane + 1), epoch};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)(member * kTupleBytes + 16 * lane), 0,
                                           kDevScope);
  }
}

// Reads member `member`'s summary; true when all eight words are this call's.
__device__ __forceinline__ bool read_tuple(const Rsrc &r, int member, uint32_t epoch, Tuple &t) {
  const uint32_t off = (uint32_t)(member * kTupleBytes);
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevScope);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kDevScope);
  const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(r, off + 32, 0, kDevScope);
  const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, off + 48, 0, kDevScope);
  t.m = __uint_as_float(a[0]);
  t.am = (int32_t)a[2];
  t.S = (double)__uint_as_float(b[0]);
  t.W = (double)__uint_as_float(b[2]);
  t.zb = __longlong_as_double((long long)((uint64_t)c[0] | ((uint64_t)c[2] << 32)));
  t.zc = (int32_t)d[0];
  t.zx = (int32_t)d[2];
  return ((a[1] == epoch) & (a[3] == epoch) & (b[1] == epoch) & (b[3] == epoch) &
          (c[1] == epoch) & (c[3] == epoch) & (d[1] == epoch) & (d[3] == epoch)) != 0;
}

__device__ __forceinline__ void write_row_outputs(const RowStatsParams &p, int64_t row,
                                                  bool greedy, const Tuple &r) {
  // H = log S - W / S, every exp value carrying a 2^32 factor
  const double H = log_d(r.S) - r.W / r.S - 32.0 * 0.69314718055994530942;
  p.argmax[row] = r.am;
  p.sample[row] = greedy ? (int64_t)r.am : (int64_t)r.zc;
  p.entropy[row] = (float)H;
}

// Exact perturbed score of column c of `row`: s from the raw logit (re-read
// from HBM), g in fp64.
__device__ __forceinline__ double exact_score(const RowStatsParams &p, int64_t row,
                                              const Recip &rc, float tc, int32_t c) {
  const float s = scale_any(p.logits[row * p.ld + c], rc, tc);
  const uint4 w = philox4x32_10((uint32_t)(c >> 2), 0u, (uint32_t)(uint64_t)row,
                                (uint32_t)((uint64_t)row >> 32), (uint32_t)p.seed,
                                (uint32_t)(p.seed >> 32));
  return (double)s + gumbel_of_word(pick(w, c & 3));
}

// The merger's work for `row`: waits for the C member summaries, merges
// them, writes the row's outputs and, with probs, the row result.
// The sample is the member winner with the largest score; when another
// member's score is within 2^-8 of it (both may be fp32 estimates, each
// within 2^-9), the close ones are rescored exactly and the largest exact
// score wins, ties to the lower column.
template <int PROBS>
__device__ __forceinline__ void merge_row(const RowStatsParams &p, int64_t row) {
  const Rsrc r = tuple_rsrc(p, row);
  const int lane = lane_id();
  Tuple acc = empty_tuple();
  double b1 = -INFINITY, b2 = -INFINITY;  // this lane's best and second-best member scores
  int32_t c1 = INT_MAX, x1 = 1;
  for (int i = lane; i < p.C; i += kWave) {
    Tuple t;
    uint32_t spins = 0;
    while (!read_tuple(r, i, p.epoch, t)) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit || call_failed(p.err_flag, p.epoch)) {
        give_up(p.err_flag, p.epoch);
        break;
      }
    }
    acc = combine(acc, t);
    if (t.zb > b1 || (t.zb == b1 && t.zc < c1)) {
      b2 = b1;
      b1 = t.zb;
      c1 = t.zc;
      x1 = t.zx;
    } else {
      b2 = fmax(b2, t.zb);
    }
  }
  Tuple m = wave_merge(acc);
  const float T = load_uniform(p.temps + slot_of(p, row));
  const bool greedy = !(T > 0.0f);
  const double zmax = wave_allreduce(b1, MaxD());
  if (!greedy && zmax != -INFINITY) {
    const double zcut = zmax - 0x1p-8;
    const uint64_t near = __ballot(b1 >= zcut);
    if (__popcll(near) == 1 && __ballot(b2 >= zcut) == 0) {
      m.zc = __builtin_amdgcn_readlane(c1, __builtin_ctzll(near));
    } else {
      const float tc = clamp_temp(T);
      const Recip rc = recip_of(tc);
      double bz = -INFINITY;
      int32_t bc = INT_MAX;
      auto consider = [&](double zrep, int32_t c, int32_t zx) {
        const double z = zx ? zrep : exact_score(p, row, rc, tc, c);
        if (z > bz || (z == bz && c < bc)) {
          bz = z;
          bc = c;
        }
      };
      if (b1 >= zcut) consider(b1, c1, x1);
      if (b2 >= zcut) {
        // two close members in this lane (rare): every member within the cut
        for (int i = lane; i < p.C; i += kWave) {
          Tuple t;
          read_tuple(r, i, p.epoch, t);
          if (t.zb >= zcut && t.zc != c1) consider(t.zb, t.zc, t.zx);
        }
      }
      const double zbx = wave_allreduce(bz, MaxD());
      m.zc = wave_allreduce(bz == zbx ? bc : INT_MAX, MinI());
    }
  }
  if (lane == 0) {
    write_row_outputs(p, row, greedy, m);
    // the row result: with probs the writers need it, without probs it only
    // paces the members
    store_row_result(p.rowres, row, __float_as_uint(m.m), __float_as_uint((float)(1.0 / m.S)), p.epoch);
  }
}

// ---------------------------------------------------------------------------
// Reduction of one chunk. On entry v holds the chunk's raw logits; on return
// v holds the exp values 2^32 exp(s - m) of the wave and every lane holds the
// wave's summary (its best score exact when `exact` is set).
// ---------------------------------------------------------------------------
// With LDSX, xbuf is the wave's LDS copy of this chunk's raw logits (kept
// until the chunk is reduced): candidates read their logits there. clist is
// the wave's LDS list of kWave candidate columns.
template <bool VEC, bool VKEYS, bool LDSX>
__device__ __forceinline__ Tuple reduce_chunk(const RowStatsParams &p, int64_t row, int32_t chunk,
                                              float4 (&v)[kQ], bool exact,
                                              const PhiloxRoundKeys &rk, const float4 *xbuf,
                                              int32_t *clist) {
  const int lane = lane_id();
  const int32_t V = p.vocab;
  const float T = load_uniform(p.temps + slot_of(p, row));
  const bool greedy = !(T > 0.0f);
  const float tc = clamp_temp(T);
  const Recip rc = recip_of_uniform(tc);
  const double rtc = rc.hi;
  const int32_t c0 = chunk * kChunkCols;
  // column of element k = 4 j + i of this lane
  auto col_of = [&](int k) -> int32_t { return c0 + 4 * ((k >> 2) * kWave + lane) + (k & 3); };

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
            float x;
            if constexpr (LDSX) x = lds_read_f32(xbuf, 4 * ((k >> 2) * kWave + lane_here()) + (k & 3));
            else x = p.logits[row * p.ld + c0 + 4 * ((k >> 2) * kWave + lane_here()) + (k & 3)];
            set_comp(v[k >> 2], k & 3, scale_dd(x, rc));
          }
        }
        mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kQ; ++j) mt = fmaxf(mt, max4(v[j]));
      }
    }
  }
  const float mw = wave_max_f32(mt);

  // ---- lowest column of the wave attaining its max ----
  // kt: this lane's first element equal to its own maximum (the Gumbel
  // bound below uses it too)
  int32_t kt = 0;
#pragma unroll
  for (int k = 4 * kQ - 1; k >= 0; --k)
    if (comp(v[k >> 2], k & 3) == mt) kt = k;
  const int32_t amw = wave_allreduce(mt == mw ? col_of(kt) : INT_MAX, MinI());

  // ---- exp values e = 2^32 exp(s - m) in place of s, and their sums ----
  // The 2^32 factor keeps every probability that survives rounding to
  // bf16/fp16 away from fp32 denormals; it cancels in every ratio.
  // d = s - m is -inf for a -inf logit (and for a masked column, or when the
  // difference overflows); then e = 0 and e d is NaN, which the wave sum of
  // W shows. Such a wave recomputes W below with d clamped to -FLT_MAX (its
  // terms are then 0), in the same order; every other wave skips the clamp.
  const float mu = (mw == -INFINITY) ? 0.0f : mw;
  float St = 0.0f, Wt = 0.0f;
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    float4 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = comp(v[j], i) - mu;
      const float ei = __builtin_amdgcn_exp2f(fmaf(d, kLog2e, 32.0f));
      St += ei;
      Wt = fmaf(ei, d, Wt);
      set_comp(e, i, ei);
    }
    v[j] = e;
  }

  // wave sums in fp32 (the summary carries them as fp32 words)
  const float Sw = wave_allreduce(St, SumF());

  // ---- Gumbel-max over the wave's columns (T > 0) ----
  // The wave reports its best perturbed score z = s + g and that column. The
  // score is an fp32 estimate (within 2^-9 of exact) unless the wave had to
  // compare candidates closer than that, or `exact` asks for it; then it is
  // the exact fp64 score. The row merge settles close calls between chunks.
  double zb = -INFINITY;
  int32_t zc = INT_MAX, zx = 1;
  if (!greedy && mw != -INFINITY) {
    const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
    const uint32_t r0 = (uint32_t)(uint64_t)row, r1 = (uint32_t)((uint64_t)row >> 32);
    // quad of j = 0. The counters are the same for every row of this wave:
    // with lane_id() the compiler keeps them (or the first Philox round's
    // products) across the row loop and, short of registers, reloads them
    // from scratch memory, and each such reload waits for the chunk copy in
    // flight.
    const uint32_t qb = (uint32_t)chunk * kChunkQuads + (uint32_t)lane_here();
    constexpr float kLn2 = 0.693147180559945309f;
    // fp32 Gumbel value -log(-log u) of a word, error below 2^-12
    auto g32 = [&](uint32_t w) { return -__builtin_amdgcn_logf(neg_log_u_f32(w)) * kLn2; };
    // The word of each lane's own maximum (column ct); the lane holding the
    // wave's argmax thereby has the argmax's word.
    const int32_t ct = col_of(kt);
    const uint32_t wt = pick(philox4x32_10((uint32_t)(ct >> 2), 0u, r0, r1, k0, k1), ct & 3);
    // a = exp(m - zlb) = -log u of the argmax's word, zlb = m + g_argmax
    const int la = __builtin_ctzll(__ballot(mt == mw && ct == amw));
    float a = neg_log_u_f32((uint32_t)__builtin_amdgcn_readlane((int)wt, la));
    // Flat waves let many columns pass the test; the expected number is
    // sum_c exp(s_c - zlb) = a sum e / 2^32. When it is large, raise zlb to
    // a lower bound of the best score among every lane's own maximum.
    if (Sw * 0x1p-32f * a > 8.0f) {
      // relative to m
      float zt = (mt != -INFINITY) ? (mt - mw) + g32(wt) - 0x1p-10f : -INFINITY;
      zt = wave_max_f32(zt);
      a = fminf(a, __builtin_amdgcn_exp2f(-zt * kLog2e) * (1.0f + 0x1p-12f));
    }
    const float kc = a * kTestMargin;
    const float ethr = kQuadSkip / a;
    // Candidate test of a column with word w and exp value e: it can reach
    // zlb only if 1 - u <= e a 2^-32, i.e. w >= 2^32 - 1/2 - e a. Tested as
    // fl32(w) >= fl32(2^32 - 512 - e kc): fl32(w) is within 128 of w, the fma
    // rounds by at most 128 and kc covers the rounding of e and a, so every
    // such column passes (a few more may). Bit 31 - k of cm is element k.
    // A quad first takes the test with its largest word and exp value: as
    // rounding is monotone, a quad that fails it holds no passing column,
    // and only the lanes of a quad that passes (rare) test its four columns.
    uint32_t cm = 0;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const float ej = max4_nonneg(v[j]);
      if (ej >= ethr) {
        const uint4 w = VKEYS ? philox4x32_10(qb + (uint32_t)(j * kWave), 0u, r0, r1, k0, k1, rk)
                              : philox4x32_10(qb + (uint32_t)(j * kWave), 0u, r0, r1, k0, k1);
        const uint32_t wm = max(max(w.x, w.y), max(w.z, w.w));
        if ((float)wm >= fmaf(-ej, kc, 4294966784.0f)) {
          cm = push4_bits_ge(cm, (float)w.x, (float)w.y, (float)w.z, (float)w.w,
                             fmaf(-v[j].x, kc, 4294966784.0f), fmaf(-v[j].y, kc, 4294966784.0f),
                             fmaf(-v[j].z, kc, 4294966784.0f), fmaf(-v[j].w, kc, 4294966784.0f));
        } else {
          cm <<= 4;
        }
      } else {
        cm <<= 4;
      }
    }
    // Every candidate gets an fp32 score relative to m: s - m from its raw
    // logit plus its fp32 Gumbel value. Each lane keeps its best two. The
    // logit comes from the chunk's LDS copy when there is one; otherwise it
    // is re-read from memory (it was just streamed, so the read normally
    // hits the cache, but the wait for it also waits for the chunk copy in
    // flight). Scoring from the exp values in registers avoids both but
    // costs more vector instructions, and measures slower.
    float za1 = -INFINITY, za2 = -INFINITY;
    int32_t cbest = INT_MAX;
    auto score = [&](int32_t c) {
      if (c < V) {
        float x;
        if constexpr (LDSX) x = lds_read_f32(xbuf, c - c0);
        else x = p.logits[row * p.ld + c];
        const uint4 w = philox4x32_10((uint32_t)(c >> 2), 0u, r0, r1, k0, k1);
        const float z = (scale(x, rtc) - mw) + g32(pick(w, c & 3));
        if (z > za1) {
          za2 = za1;
          za1 = z;
          cbest = c;
        } else {
          za2 = fmaxf(za2, z);
        }
      }
    };
    // The loop over a lane's candidates runs as often as the lane with the
    // most of them needs. When some lane has two or more and the wave has at
    // most 64, the candidates are first spread one per lane through LDS, so
    // one scoring pass serves them all (each lane then holds at most one).
    bool spread = false;
    if (__ballot(__popc(cm) >= 2) != 0) {
      int total;
      int o = wave_prefix(__popc(cm), total);
      if (total <= kWave) {
        spread = true;
        for (uint32_t c2 = cm; c2 != 0;) {
          const int k = __builtin_clz(c2);
          c2 &= ~(0x80000000u >> k);
          clist[o++] = col_of(k);
        }
        wave_lds_order();
        // (the lane number taken afresh: an address kept from before the
        // row loop would be spilled, and its reload waits for the copy)
        const int l = lane_here();
        const int32_t c = l < total ? clist[l] : INT_MAX;
        wave_lds_order();
        score(c);
      }
    }
    if (!spread) {
      for (uint32_t c2 = cm; c2 != 0;) {
        const int k = __builtin_clz(c2);
        c2 &= ~(0x80000000u >> k);
        score(col_of(k));
      }
    }
    // Only candidates within 2^-8 of the wave's best estimate can win.
    const float zmax = wave_max_f32(za1);
    const float zcut = zmax - 0x1p-8f;
    const uint64_t near = __ballot(za1 >= zcut);
    if (!exact && __popcll(near) == 1 && __ballot(za2 >= zcut) == 0) {
      zc = __builtin_amdgcn_readlane(cbest, __builtin_ctzll(near));
      zb = (double)mw + (double)zmax;
      zx = 0;
    } else {
      // exact fp64 scores of the candidates within the cut
      double bz = -INFINITY;
      int32_t bc = INT_MAX;
      auto score_exact = [&](int32_t c) {
        if (c < V) {
          const double z = exact_score(p, row, rc, tc, c);
          if (z > bz || (z == bz && c < bc)) {
            bz = z;
            bc = c;
          }
        }
      };
      if (za1 >= zcut) score_exact(cbest);
      if (za2 >= zcut) {  // (never after spreading: one candidate per lane)
        for (uint32_t c2 = cm; c2 != 0;) {
          const int k = __builtin_clz(c2);
          c2 &= ~(0x80000000u >> k);
          if (col_of(k) != cbest) score_exact(col_of(k));
        }
      }
      zb = wave_allreduce(bz, MaxD());
      zc = wave_allreduce(bz == zb ? bc : INT_MAX, MinI());
      zx = 1;
    }
  }

  float Ww = wave_allreduce(Wt, SumF());
  if (Ww != Ww) {
    // Some e d was 0 times -inf: W again, with d clamped, from the logits
    // (the LDS copy of the chunk, else memory; rare: -inf logits, the row
    // end, values near the fp32 limit).
    const int32_t left = V - c0 - 4 * lane_here();
    Wt = 0.0f;
#pragma unroll
    for (int j = 0; j < kQ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t k = 4 * j * kWave + i;  // column c0 + 4 lane + k
        float x = -INFINITY;
        if (k < left) {
          if constexpr (LDSX) x = lds_read_f32(xbuf, 4 * lane_here() + k);
          else x = p.logits[row * p.ld + c0 + 4 * lane_here() + k];
        }
        const float s = (T == 1.0f || x == -INFINITY) ? x : scale_any(x, rc, tc);
        Wt = fmaf(comp(v[j], i), fmaxf(s - mu, -FLT_MAX), Wt);
      }
    Ww = wave_allreduce(Wt, SumF());
  }

  Tuple t;
  t.m = mw;
  t.am = amw;
  t.S = (double)Sw;
  t.W = (double)Ww;
  t.zb = zb;
  t.zc = zc;
  t.zx = zx;
  return t;
}

// From a chunk's exp values e = 2^32 exp(s - mw) to probabilities
// p = e exp(mw - m) / S, S carrying the same 2^32 factor: p = e f with
// f = exp(mw - m) / S. For a chunk far below the row maximum f leaves the
// fp32 normal range (below 2^-126 once mw - m is under about -65 + log S)
// while its probabilities can still be nonzero bf16 / fp16 values (down to
// 2^-133, s - m near -92), so there the factor is lifted by 2^96 and the
// product brought back with an exact power-of-two multiply:
// p = (e f') 2^-96, f' = 2^96 f, rounded once into the subnormal range.
struct ProbScale {
  float f;
  bool lifted;
};

__device__ __forceinline__ ProbScale prob_scale(float mw, float m, float inv_s) {
  if (mw == -INFINITY) return {0.0f, false};
  const float d = fmaxf(mw - m, -FLT_MAX) * kLog2e;  // <= 0
  const float f = __builtin_amdgcn_exp2f(d) * inv_s;
  if (f >= 0x1p-126f) return {f, false};
  // 2^64 exp(mw - m) stays normal down to mw - m = -131, past which every
  // probability of the chunk is below 2^-189; inv_s 2^32 = 2^32 / S <= 1
  return {__builtin_amdgcn_exp2f(d + 64.0f) * (inv_s * 0x1p32f), true};
}

template <int PROBS, bool VEC>
__device__ __forceinline__ void write_probs(const RowStatsParams &p, int64_t row, int32_t chunk,
                                            const float4 (&e)[kQ], ProbScale ps) {
  const int lane = lane_id();
  const int32_t c0 = chunk * kChunkCols;
  const Rsrc w = make_rsrc(reinterpret_cast<uint16_t *>(p.probs) + row * (int64_t)p.vocab + c0,
                           2u * (uint32_t)min(p.vocab - c0, kChunkCols));
  auto pack = [](float a, float b) {
    return (PROBS == 1) ? pack_bf16x2(a, b) : pack_fp16x2(a, b);
  };
  auto store = [&](int j, const u32x2 &pk) {
    if constexpr (VEC) {
      __builtin_amdgcn_raw_buffer_store_b64(pk, w, 8u * lane, 8 * kWave * j, kNonTemporal);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk[i >> 1] >> (16 * (i & 1))), w, 8u * lane,
                                              8 * kWave * j + 2 * i, kNonTemporal);
    }
  };
  const float sc = ps.f;
  if (!ps.lifted) {
#pragma unroll
    for (int j = 0; j < kQ; ++j)
      store(j, u32x2{pack(e[j].x * sc, e[j].y * sc), pack(e[j].z * sc, e[j].w * sc)});
  } else {
    constexpr float kDown = 0x1p-96f;
#pragma unroll
    for (int j = 0; j < kQ; ++j)
      store(j, u32x2{pack((e[j].x * sc) * kDown, (e[j].y * sc) * kDown),
                     pack((e[j].z * sc) * kDown, (e[j].w * sc) * kDown)});
  }
}

// ---------------------------------------------------------------------------
// The kernel. Global wave gw belongs to group gw / C as member gw % C: the
// group reduces one row at a time (rows from a RowDealer), the member chunk
// `member` of each. The merger of the group's n-th row is member n % C; it merges
// row n after reducing row n + kMergeLag. Before publishing row n, every
// member waits for the result of row n - kLag (normally there for a whole
// chunk): with probs it needs it to write that row's probabilities, and
// without probs the wait keeps the waves of a SIMD in step (otherwise the
// older wave, favoured by the issue arbiter, would finish early and leave
// the SIMD half idle). A merge delays its merger's next chunks; the merger
// of a later row waits for such a late chunk only when the delay exceeds
// kMergeLag chunk periods. With probs, each row of lag keeps the row's exp
// values in registers, so the lags stay short there.
// ---------------------------------------------------------------------------
template <int PROBS, bool VEC>
__global__ __launch_bounds__(kThreads, PROBS ? 2 : 4) void rowstats_kernel(RowStatsParams p) {
  constexpr int kMergeLag = PROBS ? 1 : 2;
  constexpr int kLag = kMergeLag + 2;
  // one LDS buffer of one chunk per wave (vector path): the next chunk is
  // copied in as soon as the current one has been read into registers
  // With probs (2 waves per SIMD, LDS to spare) each wave has two buffers:
  // the chunk being reduced stays in one while the next is copied into the
  // other, so its candidates read their logits from LDS.
  constexpr int kBufs = (VEC && PROBS != 0) ? 2 : 1;
  __shared__ float4 stage[VEC ? kWaves * kChunkQuads * kBufs : 1];
  // Gumbel candidates spread one per lane (kWave columns per wave)
  __shared__ int32_t clists[kWaves * kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int gw = (int)blockIdx.x * kWaves + wave;
  // the next call's row-claim counter starts at zero
  if (gw == 0 && lane_id() == 0) p.counters[(p.epoch + 1) & 1] = 0u;
  const int group = gw / p.C;
  const int member = gw - group * p.C;
  if (group >= p.n_groups || group >= p.rows) return;
  const int32_t chunk = member;
  const bool leader = member == 0;
  // with probs, the Philox round keys live in vector registers (there are
  // free ones there); without, each call steps them in scalar registers
  const PhiloxRoundKeys rk =
      philox_round_keys_v(PROBS ? (uint32_t)p.seed : 0u, PROBS ? (uint32_t)(p.seed >> 32) : 0u);
  RowDealer d;
  d.ring = p.rings + (int64_t)group * (kRingBytes / 8);
  d.counter = p.counters + (p.epoch & 1);
  d.limit = p.rows;
  d.first = (int64_t)kDealAhead * p.n_groups;
  d.group = group;
  d.G = p.n_groups;
  d.epoch = p.epoch;
  float4 *const buf0 = stage + (VEC ? wave * kChunkQuads * kBufs : 0);
  float4 *const buf1 = buf0 + (kBufs - 1) * kChunkQuads;
  // Copies the chunk of row `row` into the wave's buffer. Past the last row
  // (row < 0) the copy still issues (through a zero-size descriptor: nothing
  // is read, the buffer gets zeros), so every path issues the same
  // operations and the compiler can count them exactly.
  const uint32_t bytes = chunk_bytes(chunk * kChunkCols, p.vocab);
  auto copy_chunk = [&](float4 *buf, int64_t row) {
    chunk_copy_bytes(buf, row >= 0 ? p.logits + row * p.ld + chunk * kChunkCols : p.logits,
                     row >= 0 ? bytes : 0u);
  };

  float4 cur[kQ];
  // exp values and wave maxima of rows n - 1, n - 2, n - 3 (with probs)
  float4 p1[PROBS ? kQ : 1], p2[PROBS ? kQ : 1], p3[PROBS ? kQ : 1];
  float m1 = -INFINITY, m2 = -INFINITY, m3 = -INFINITY;
  // rows of iterations n (row), n + 1 and n - 1 .. n - kLag (hist)
  int64_t row = group, row_next = d.static_pos(1);
  int64_t hist[kLag];
#pragma unroll
  for (int i = 0; i < kLag; ++i) hist[i] = -1;
  int mturn = 0;  // (n - kMergeLag) % C
  if constexpr (VEC) copy_chunk(buf0, row);
  for (int n = 0; row >= 0; ++n) {
    const int64_t pace_row = hist[kLag - 1];
    // row result of row n - kLag, written by its merger more than a chunk
    // ago (loaded every time so that no path leaves the register waiting on
    // a load), the ring slot of row n + 2 and (member 0) a claim
    u32x4 rr = load_row_result(p.rowres, pace_row >= 0 ? pace_row : row);
    u32x4 slot = d.load_slot(n + 2);
    uint32_t claim = 0;
    if (leader) claim = d.claim();
    compiler_fence();
    if constexpr (VEC) {
      // The copy of this row's chunk was followed, in the previous row, by
      // (member 0) a ring post, with probs (once rows are kLag behind) eight
      // probs stores, the summary store, and in this row by the row-result
      // and slot loads; at most that many operations may still be pending.
      if (n == 0) wait_vm<0>();
      else if (PROBS != 0 && n > kLag) {
        if (leader) wait_vm<12>();
        else wait_vm<11>();
      } else {
        if (leader) wait_vm<4>();
        else wait_vm<3>();
      }
      lds_read_chunk(cur, (n & 1) ? buf1 : buf0);
      compiler_fence();
      copy_chunk((n & 1) ? buf0 : buf1, row_next);
      compiler_fence();
    } else {
      chunk_load(cur, p.logits + row * p.ld, chunk * kChunkCols, p.vocab);
    }
    const Tuple t = reduce_chunk<VEC, PROBS != 0, kBufs == 2>(p, row, chunk, cur, false, rk,
                                                              (n & 1) ? buf1 : buf0,
                                                              clists + wave * kWave);
    // The empty statement consumes the loads issued before the copy on
    // every path, so the wait for them is placed here, exactly, and does not
    // wait for the copy.
    __asm__ volatile("" ::"v"(rr), "v"(slot), "v"(claim));
    compiler_fence();
    const int64_t row_after =
        n + 2 < kDealAhead ? d.static_pos(n + 2) : d.slot_pos(slot, n + 2, p.err_flag);
    if (leader) d.post(n + kDealAhead, d.claimed_pos(claim));
    // row n - kLag first: waiting for its result then does not wait for the
    // summary store below
    if (pace_row >= 0) {
      rr = wait_row_result(p.rowres, pace_row, rr, p.epoch, p.err_flag);
      if constexpr (PROBS != 0)
        write_probs<PROBS, VEC>(p, pace_row, chunk, p3,
                                prob_scale(m3, __uint_as_float(rr[0]), __uint_as_float(rr[2])));
    }
    compiler_fence();
    publish_tuple(tuple_rsrc(p, row), member, t, p.epoch);
    compiler_fence();
    if (n >= kMergeLag) {
      if (mturn == member) merge_row<PROBS>(p, hist[kMergeLag - 1]);
      if (++mturn == p.C) mturn = 0;
    }
    if constexpr (PROBS != 0) {
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        p3[j] = p2[j];
        p2[j] = p1[j];
        p1[j] = cur[j];
      }
      m3 = m2;
      m2 = m1;
      m1 = t.m;
    }
#pragma unroll
    for (int i = kLag - 1; i > 0; --i) hist[i] = hist[i - 1];
    hist[0] = row;
    row = row_next;
    row_next = row_after;
  }
  // the last kMergeLag rows (fewer if the group has fewer rows)
#pragma unroll
  for (int i = kMergeLag - 1; i >= 0; --i) {
    if (hist[i] < 0) continue;
    if (mturn == member) merge_row<PROBS>(p, hist[i]);
    if (++mturn == p.C) mturn = 0;
  }
  if constexpr (PROBS != 0) {
    // the last kLag rows' probabilities (kLag = 3 with probs)
    static_assert(PROBS == 0 || kLag == 3, "three rows of exp values are kept");
    auto finish = [&](int64_t r, const float4 (&e)[kQ], float mw) {
      if (r < 0) return;
      const u32x4 v = wait_row_result(p.rowres, r, load_row_result(p.rowres, r), p.epoch, p.err_flag);
      write_probs<PROBS, VEC>(p, r, chunk, e, prob_scale(mw, __uint_as_float(v[0]), __uint_as_float(v[2])));
    };
    finish(hist[2], p3, m3);
    finish(hist[1], p2, m2);
    finish(hist[0], p1, m1);
  }
}

// ---------------------------------------------------------------------------
// Host side: occupancy query and launch (called by the C ABI).
// ---------------------------------------------------------------------------
template <int PROBS, bool VEC>
static const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&rowstats_kernel<PROBS, VEC>);
}

static const void *select_kernel(int probs_dtype, bool vec) {
  if (vec) {
    switch (probs_dtype) {
      case 1: return kernel_ptr<1, true>();
      case 2: return kernel_ptr<2, true>();
      default: return kernel_ptr<0, true>();
    }
  }
  switch (probs_dtype) {
    case 1: return kernel_ptr<1, false>();
    case 2: return kernel_ptr<2, false>();
    default: return kernel_ptr<0, false>();
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
  return hipLaunchCooperativeKernel(select_kernel(probs_dtype, p.vec_ok != 0), dim3(grid),
                                    dim3(kThreads), args, 0, stream);
}

}  // namespace rowstats
