// correct.hip -- exact correction of the selected tokens, then the merge of
// everything into the output (JetFire README, introduction: the top-k tokens
// get a high-precision correction; here from the fp16 shadow rows).
//
// With the merged approximate state (M, L, A) of head h over all tokens (log2
// units), the selected set S, exact logits s_t and approximate ones s_hat_t:
//   m' = max(M, max_S s_t)
//   l' = 2^(M-m') (L - sum_S 2^(s_hat_t - M))        + sum_S 2^(s_t - m')
//   a' = 2^(M-m') (A - sum_S 2^(s_hat_t - M) V_hat_t) + sum_S 2^(s_t - m') V_t
//   out = a' / l'
// i.e. the selected tokens' approximate terms leave the sums and their exact
// terms enter, then everything is renormalised.  When every token is selected
// the approximate state is not used at all.
//
// Two launches:
//   chunk   one workgroup per (unit, 32 selected tokens): exact and
//           approximate logits of the chunk's tokens for the unit's G query
//           heads (8 threads per token), then per head the chunk's exact state
//           (m, l, sum 2^(s-m) V) and approximate state (same with s_hat,
//           V_hat), one thread per channel for the value sums (their loads are
//           issued before the logits are computed);
//   combine one thread per (query head, channel): online-softmax merges of the
//           scan's split states and of the chunk states (every load of a
//           record independent of the others, batched), then the formula
//           above.
#include <mutex>

#include "bkv_internal.h"
#include "correct_lane.h"
#include "quant_lane.h"

namespace bkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Running softmax state: max m (log2 units), scaled sums a and l.
struct Online {
  float m = -INFINITY, a = 0.f, l = 0.f;
  __device__ void add(float mj, float lj, float aj) {  // branch-free: loads stay batched
    const float mn = fmaxf(m, mj);
    const float ref = (mn == -INFINITY) ? 0.f : mn;  // both -inf: factors 0, nothing changes
    const float f0 = __builtin_amdgcn_exp2f(m - ref), f1 = __builtin_amdgcn_exp2f(mj - ref);
    a = fmaf(a, f0, aj * f1);
    l = fmaf(l, f0, lj * f1);
    m = mn;
  }
  // the sums expressed relative to the max `ref` (>= m up to rounding)
  __device__ float scale_to(float ref) const { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - ref); }
};

constexpr int kRecBatchMax = 16;  // records per batch: 16, or 8 when every list fits 8

// Records j0..j0+kRecBatch-1 of a set (max m[j*sm], denominator l[j*sm],
// value v[j*sv]); past cnt they are empty.  Loads are clamped and
// unconditional so that a whole batch is in flight at once.  The batch's
// maxima and denominators, the same for every lane, arrive as one vector
// load each (lane i % kRecBatch takes record j0 + i % kRecBatch) and are
// read out of those lanes: as scalar loads they were 2 * kRecBatch loads
// per set that the scalar unit's few outstanding requests serialise.
template <int kRecBatch>
struct RecBatch {
  float m[kRecBatch], l[kRecBatch], v[kRecBatch];
  __device__ void load(const float* __restrict__ pm_, const float* __restrict__ pl_, const float* __restrict__ pv,
                       size_t sm, size_t sv, int cnt, int j0) {
    const size_t jl = (size_t)max(min(j0 + (int)(__builtin_amdgcn_workitem_id_x() % kRecBatch), cnt - 1), 0);
    const float mv = pm_[jl * sm], lv = pl_[jl * sm];
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      const size_t j = (size_t)max(min(j0 + i, cnt - 1), 0);
      v[i] = pv[j * sv];
    }
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      m[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), i));
      l[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), i));
    }
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) {
      const bool ok = j0 + i < cnt;
      m[i] = ok ? m[i] : -INFINITY;
      l[i] = ok ? l[i] : 0.f;
      v[i] = ok ? v[i] : 0.f;
    }
  }
  __device__ void into(Online& st) const {
#pragma unroll
    for (int i = 0; i < kRecBatch; ++i) st.add(m[i], l[i], v[i]);
  }
};

// One workgroup per (b, query head): kCombineGroups groups of one thread per
// channel take the record batches in turn (so long record lists are read in
// parallel), then the first group merges the groups' states.  hx (may be
// null): the exact state of the selected tokens per (b, query head),
// {m, l, a[0..D)}, in place of the chunk records' exact parts.
// (One group when every list fits one batch: no barrier, no LDS.)
template <int kCombineGroups, int kRecBatch = kRecBatchMax>
__global__ __launch_bounds__(kHeadDim * kCombineGroups) void combine_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                           const float* __restrict__ pacc, const float* __restrict__ cs,
                                                           const float* __restrict__ hx, float* __restrict__ out,
                                                           SeqArg lens, int Hq, int nsplit, int nchunk, int k,
                                                           int rest, int rec_tokens) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x & (kHeadDim - 1);
  // the group is the same in a whole wave: kept scalar, so the record loop and
  // the loads of each record's max and denominator stay scalar too
  const int grp = (kCombineGroups > 1) ? __builtin_amdgcn_readfirstlane(threadIdx.x / kHeadDim) : 0;
  const int n = lens.v[b];
  const size_t rec = (size_t)b * Hq + h;
  float* o = out + rec * kHeadDim;
  if (n == 0) {
    if (grp == 0) o[c] = 0.f;
    return;
  }
  const int kk = min(k, n);
  const int nc = (kk + rec_tokens - 1) / rec_tokens;  // records (each of rec_tokens row entries)
  const float* ps = cs + rec * (size_t)nchunk * kCsStride;
  // exact state of the selected tokens, approximate state of every token and
  // approximate terms of the selected tokens; a batch's loads of all three
  // are issued before any is used
  const int nap = (kk < n) ? nsplit : 0;  // every token selected: the scan state is not needed
  const int nsel = (kk < n && !rest) ? nc : 0;  // rest: the split states already leave S out
  Online ex, ap, sel;
  const int nex = hx ? 0 : nc;  // exact records from the chunks
  if (hx && grp == 0) {
    const float* x = hx + rec * kStateFloats;
    ex.add(x[0], x[1], x[2 + c]);
  }
  for (int j0 = grp * kRecBatch; j0 < max(nc, nap); j0 += kCombineGroups * kRecBatch) {
    RecBatch<kRecBatch> be, ba, bs;
    be.load(ps, ps + 1, ps + 4 + c, kCsStride, kCsStride, nex, j0);
    ba.load(pm + rec * nsplit, pl + rec * nsplit, pacc + rec * nsplit * kHeadDim + c, 1, kHeadDim, nap, j0);
    bs.load(ps + 2, ps + 3, ps + 4 + kHeadDim + c, kCsStride, kCsStride, nsel, j0);
    be.into(ex);
    ba.into(ap);
    bs.into(sel);
  }
  if constexpr (kCombineGroups > 1) {
  // the other groups' states to the first group
  __shared__ float s_st[kCombineGroups - 1][3][3][kHeadDim];  // [group - 1][ex/ap/sel][m/l/a][c]
  if (grp > 0) {
    float* d = &s_st[grp - 1][0][0][c];
    d[0 * kHeadDim] = ex.m, d[1 * kHeadDim] = ex.l, d[2 * kHeadDim] = ex.a;
    d[3 * kHeadDim] = ap.m, d[4 * kHeadDim] = ap.l, d[5 * kHeadDim] = ap.a;
    d[6 * kHeadDim] = sel.m, d[7 * kHeadDim] = sel.l, d[8 * kHeadDim] = sel.a;
  }
  __syncthreads();
  if (grp > 0) return;
#pragma unroll
  for (int g = 0; g < kCombineGroups - 1; ++g) {
    ex.add(s_st[g][0][0][c], s_st[g][0][1][c], s_st[g][0][2][c]);
    ap.add(s_st[g][1][0][c], s_st[g][1][1][c], s_st[g][1][2][c]);
    sel.add(s_st[g][2][0][c], s_st[g][2][1][c], s_st[g][2][2][c]);
  }
  }
  if (kk == n) {
    o[c] = ex.a / ex.l;
    return;
  }
  if (kk == 0) {
    o[c] = ap.a / ap.l;
    return;
  }
  if (rest) {  // a plain merge of the unselected tokens' state and the selected tokens' exact state
    const float mp = fmaxf(ap.m, ex.m);
    const float fa = __builtin_amdgcn_exp2f(ap.m - mp);
    const float fe = (ex.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ex.m - mp);
    o[c] = (fa * ap.a + fe * ex.a) / (fa * ap.l + fe * ex.l);
    return;
  }
  const float M = ap.m;
  const float fs = sel.scale_to(M);
  const float A = ap.a - fs * sel.a, L = fmaxf(ap.l - fs * sel.l, 0.f);
  const float mp = fmaxf(M, ex.m);
  const float fa = __builtin_amdgcn_exp2f(M - mp), fe = __builtin_amdgcn_exp2f(ex.m - mp);
  o[c] = (fa * A + fe * ex.a) / (fa * L + fe * ex.l);
}

// ---- exact terms of long rows (whole blocks of tokens) --------------------------
// One workgroup per (unit, record of kRowRec row entries), four waves, each
// taking 16-entry tiles of the record in turn with a softmax state of its own:
//  * logits on v_mfma_f32_16x16x32_f16: A = the tile's fp16 shadow key rows,
//    K-step ks taking channels 32ks .. 32ks+31, lane (r, kb) channels
//    32ks + 8kb .. +7 of entry r's token (each of the four loads covers 64
//    contiguous bytes of 16 rows); B = column n holding query head n mod G
//    on the same channels.  D leaves entry 4kb+i's logit of head n mod G in
//    lane (n, kb).
//  * weights and the running max per head go through a per-wave LDS slot;
//  * P.V on the VALU in fp32: lane (p, q) reads channels 8p .. 8p+7 of the
//    shadow value rows of entries 4j + q (16 bytes each) and accumulates all
//    G heads.
// Entries < 0 or >= len are left out.  The record's exact part (m, l and the
// value sums, log2 units) is written; its approximate part comes from the
// scan's launch over the same rows.
constexpr int kRowWaves = 4;

__device__ inline float wmax16(float x) {  // max over the lanes n, n+16, n+32, n+48
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wsum16(float x) {  // sum over the lanes n, n+16, n+32, n+48
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int G>
__global__ __launch_bounds__(64 * kRowWaves) void exact_rows_kernel(
    const uint16_t* __restrict__ k_shadow, const uint16_t* __restrict__ v_shadow, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ idx, float* __restrict__ cs, SeqArg lens, int Hq, int Hkv, int cap, int row,
    int nchunk) {
  const int u = blockIdx.y, rec_i = blockIdx.x;
  const int b = u / Hkv, kvh = u - b * Hkv;
  const int n_len = lens.v[b];
  const int kk = min(row, n_len);
  const int r_begin = rec_i * kRowRec;
  if (r_begin >= kk) return;  // the combine reads only the records below kk
  const int r_end = min(kk, r_begin + kRowRec);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kb = lane >> 4;
  const size_t head0 = (size_t)b * Hq + (size_t)kvh * G;
  const int32_t* rowp = idx + (size_t)u * row;
  const uint16_t* ksh = k_shadow + (size_t)u * cap * kHeadDim;
  const uint16_t* vsh = v_shadow + (size_t)u * cap * kHeadDim;
  const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;

  // B operands: column n = head n mod G, K-step ks = channels 32ks + 8kb .. +7
  half8 bq[4];
  {
    const uint16_t* qr = q + (head0 + (size_t)(n % G)) * kHeadDim + 8 * kb;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bq[ks] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(qr + 32 * ks));
  }

  __shared__ int s_row[kRowRec];           // the record's tokens (-1: left out)
  __shared__ float s_p[kRowWaves][16][G];  // a tile's weights, per wave
  __shared__ float s_f[kRowWaves][G];      // the factor of the running sums, per wave
  __shared__ float s_ml[kRowWaves][2][G];  // each wave's final max and denominator
  __shared__ float s_acc[kRowWaves][G][kHeadDim];

  const int pc = lane & 15, qs = lane >> 4;  // P.V: channels 8pc .. 8pc+7, entries 4j + qs of a tile
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // of head n mod G (the same in the four lanes of a column)

  // The record's tokens, once, into LDS: a tile's addresses then depend on
  // no global load (a wait for one would also wait for the loads of the tile
  // in flight before it).
  for (int i = tid; i < kRowRec; i += 64 * kRowWaves) {
    const int e = r_begin + i;
    const int t = (e < r_end) ? rowp[e] : -1;
    s_row[i] = (t >= 0 && t < n_len) ? t : -1;
  }
  __syncthreads();
  // A tile's loads (masked entries read token 0's rows, in range; they get
  // weight 0): the key rows of entries e0 + r for the logits, the value rows
  // of entries e0 + 4j + qs for P.V.
  struct Tile {
    int tr;
    uint4 ka[4];
    int tv[4];
    uint4 va[4];
  };
  auto load = [&](Tile& T, int e0) {
    T.tr = s_row[e0 - r_begin + n];  // (entries past r_end are -1)
    const uint16_t* kr = ksh + (size_t)max(T.tr, 0) * kHeadDim + 8 * kb;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) T.ka[ks] = *reinterpret_cast<const uint4*>(kr + 32 * ks);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      T.tv[j] = s_row[e0 - r_begin + 4 * j + qs];
      T.va[j] = *reinterpret_cast<const uint4*>(vsh + (size_t)max(T.tv[j], 0) * kHeadDim + 8 * pc);
    }
  };
  auto tile = [&](const Tile& T) {
    floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, T.ka[ks]), bq[ks], d, 0, 0, 0);
    // entry 4kb+i's logit of head n mod G is d[i] (masked entries: -inf)
    float lg[4], mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = __shfl(T.tr, 4 * kb + i);  // (lane 4kb+i holds entry 4kb+i's token)
      lg[i] = (t >= 0) ? d[i] * sm2 : -INFINITY;
      mt = fmaxf(mt, lg[i]);
    }
    mt = wmax16(mt);
    const float m_new = fmaxf(m_run, mt);
    const float ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float f = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - ref);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(lg[i] - ref);
      ls += p;
      if (n < G) s_p[wv][4 * kb + i][n] = p;
    }
    l_run = fmaf(l_run, f, wsum16(ls));
    m_run = m_new;
    if (n < G && kb == 0) s_f[wv][n] = f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float fh = s_f[wv][h];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= fh;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t vw[4] = {T.va[j].x, T.va[j].y, T.va[j].z, T.va[j].w};
      float v[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[2 * c] = h2f((uint16_t)(vw[c] & 0xFFFFu));
        v[2 * c + 1] = h2f((uint16_t)(vw[c] >> 16));
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = s_p[wv][4 * j + qs][h];  // (0 for a masked entry)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(p, v[c], acc[h][c]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // the wave's tiles e0 = r_begin + 16 (wv + 4i), one tile's loads ahead (two
  // register sets taken in turn: no copies of registers with loads in flight)
  constexpr int kStride = 16 * kRowWaves;
  int e0 = r_begin + 16 * wv;
  Tile ta, tb;
  if (e0 < r_end) load(ta, e0);
  while (e0 < r_end) {
    if (e0 + kStride < r_end) load(tb, e0 + kStride);
    tile(ta);
    e0 += kStride;
    if (e0 >= r_end) break;
    if (e0 + kStride < r_end) load(ta, e0 + kStride);
    tile(tb);
    e0 += kStride;
  }

  // the wave's state: sums over its four entry slots, then into LDS
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = wsum16(acc[h][c]);
  if (qs == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wv][h][8 * pc + c] = acc[h][c];
  }
  if (n < G && kb == 0) {
    s_ml[wv][0][n] = m_run;
    s_ml[wv][1][n] = l_run;
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += 64 * kRowWaves) {
    const int h = e / kHeadDim, c = e - h * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kRowWaves; ++x) M = fmaxf(M, s_ml[x][0][h]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int x = 0; x < kRowWaves; ++x) {
        const float fx = (s_ml[x][0][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_ml[x][0][h] - M);
        a = fmaf(fx, s_acc[x][h][c], a);
        l = fmaf(fx, s_ml[x][1][h], l);
      }
    }
    float* rec = cs + ((head0 + h) * nchunk + rec_i) * kCsStride;
    rec[4 + c] = a;
    if (c == 0) {
      rec[0] = M;
      rec[1] = l;
    }
  }
}

// EX = false: only the approximate terms (the exact state comes from
// elsewhere, see qattn_correct_hybrid); the shadow rows are not read.
// AP = false: only the exact terms (the approximate state already leaves the
// selected tokens out, see qattn_decode_unselected); the packed cache is not
// read.
// Q8: the approximate logits take the INT8 query of the scan (quant_lane.h).
// KF: the key format -- 1: MXFP4 codes (E2M1 numbers, one power-of-two scale
// per group of 32, no zero point) against the fp16 query; 2: MXFP4 codes
// with E8M0 scales against the MXFP4 query (the scan's FP4 product).
template <int KB, int VB, int G, bool EX, bool AP = true, bool Q8 = false, int KF = 0>
__global__ __launch_bounds__(256) void chunk_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const uint32_t* __restrict__ k_meta, const uint32_t* __restrict__ v_meta,
    const uint16_t* __restrict__ k_shadow, const uint16_t* __restrict__ v_shadow,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, float* __restrict__ cs, SeqArg lens, int Hq,
    int Hkv, int cap, int k, int nchunk, int mshift) {
  const int u = blockIdx.y;
  const int chunk = blockIdx.x;
  const int b = u / Hkv;
  const int kvh = u - b * Hkv;
  const int n = lens.v[b];
  const int kk = min(k, n);
  const int tid = threadIdx.x;
  const size_t head0 = (size_t)b * Hq + (size_t)kvh * G;
  const int ip0 = chunk * kCorrChunk;
  if (ip0 >= kk) return;  // the combine reads only the chunks below kk
  const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;

  __shared__ uint4 s_qh[G][kHeadDim / 8];  // the query rows as fp16 pairs
  __shared__ float s_qs[G][kHeadDim / 16];  // sums of 16-channel runs of the query rows
  __shared__ uint4 s_q8h[Q8 ? G : 1][kHeadDim / 8];   // Q8: the codes q' as fp16 pairs
  __shared__ float s_q8s[Q8 ? G : 1][kHeadDim / 16];  // Q8: s * (sum of q' over a 16-channel run)
  __shared__ float s_q8c[Q8 ? G : 1][kHeadDim / 16];  // Q8: the scale s of the run's group
  // key format 2: the query's E2M1 codes as fp16 patterns (value * 2^-14), and
  // 2^(Xq + 28) per 16-channel run
  constexpr bool kF2 = KF == 2;
  __shared__ uint4 s_q4h[kF2 ? G : 1][kHeadDim / 8];
  __shared__ float s_q4c[kF2 ? G : 1][kHeadDim / 16];
  __shared__ int s_t[kCorrChunk];
  __shared__ float s_lg[2][kCorrChunk][G];  // logits, log2 units: [exact/approx]
  __shared__ float s_w[2][kCorrChunk][G];   // weights
  __shared__ float s_mx[2][G];
  __shared__ float s_part[2][2][G][kHeadDim];  // [exact/approx][half][h][c]

  {  // the query rows and the chunk's token indices, both loads issued at once
    const uint4 w = reinterpret_cast<const uint4*>(q + head0 * kHeadDim)[tid % (G * kHeadDim / 8)];
    const int ii = ip0 + (tid & (kCorrChunk - 1));
    const int tv = idx[(size_t)u * k + min(ii, kk - 1)];
    if (tid < G * kHeadDim / 8) {
      (&s_qh[0][0])[tid] = w;
      // 8 fp16 per thread; two neighbours make a 16-channel run
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      float r = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) r += h2f((uint16_t)(ww[j] & 0xFFFFu)) + h2f((uint16_t)(ww[j] >> 16));
      r += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xB1, 0xF, 0xF, true));  // + neighbour
      if ((tid & 1) == 0) (&s_qs[0][0])[tid >> 1] = r;
      if constexpr (Q8) {
        // a group is 4 << mshift neighbouring threads (whole waves take part)
        float x[8];
        halves8(w, x);
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
        for (int m = 1; m < (4 << mshift); m <<= 1)
          a = fmaxf(a, __int_as_float(__builtin_amdgcn_ds_bpermute(((tid & 63) ^ m) << 2, __float_as_int(a))));
        const float sc = query_scale_i8(a);
        uint32_t pk[4];
        int cs8 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c0 = query_code_i8(x[2 * j], sc), c1 = query_code_i8(x[2 * j + 1], sc);
          cs8 += c0 + c1;
          const half2_t hp = {(_Float16)(float)c0, (_Float16)(float)c1};
          pk[j] = __builtin_bit_cast(uint32_t, hp);
        }
        (&s_q8h[0][0])[tid] = (uint4){pk[0], pk[1], pk[2], pk[3]};
        cs8 += __builtin_amdgcn_mov_dpp(cs8, 0xB1, 0xF, 0xF, true);
        if ((tid & 1) == 0) {
          (&s_q8s[0][0])[tid >> 1] = sc * (float)cs8;
          (&s_q8c[0][0])[tid >> 1] = sc;
        }
      }
      if constexpr (kF2) {
        // 8 channels per thread, a quad per 32-channel quarter (whole waves)
        float x[8];
        halves8(w, x);
        uint32_t code[8];
        const int X = (int)quantise_lane_e8(x, code) - 127;
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c0 = code[2 * j], c1 = code[2 * j + 1];
          pk[j] = ((c0 & 7u) << 9) | ((c0 & 8u) << 12) | ((c1 & 7u) << 25) | ((c1 & 8u) << 28);
        }
        (&s_q4h[0][0])[tid] = (uint4){pk[0], pk[1], pk[2], pk[3]};
        if ((tid & 1) == 0) (&s_q4c[0][0])[tid >> 1] = __builtin_amdgcn_ldexpf(1.0f, X + 28);
      }
    }
    if (tid < kCorrChunk) s_t[tid] = (ii < kk && tv >= 0 && tv < n) ? tv : -1;
  }
  __syncthreads();

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  const uint32_t* kmeta = k_meta + (size_t)u * (kF2 ? 1 : meta_planes(mshift)) * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * meta_planes(mshift) * cap;
  const uint16_t* ksh = k_shadow + (size_t)u * cap * kHeadDim;
  const uint16_t* vsh = v_shadow + (size_t)u * cap * kHeadDim;

  // ---- loads: the keys of the logits, then the values; all unconditional (an
  // empty slot reads token 0, always present when a chunk runs, and is masked
  // later) so that every load is in flight before the first is needed -------
  const int tl = tid >> 3;
  const int part = tid & 7;
  const int t_sel = s_t[tl];
  KeyRun<KB, EX, AP, KF> kr;
  kr.load(ksh, kbase, kmeta, cap, max(t_sel, 0), part, mshift);
  // value loads: one thread per (channel, half of the chunk)
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  constexpr int kHalf = kCorrChunk / 2;
  uint16_t vx16[kHalf];
  ValueCode<VB> vcd[kHalf];
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    const int t = max(s_t[half * kHalf + j], 0);
    if constexpr (AP) vcd[j].load(vbase, vmeta, cap, t, c, mshift);
    vx16[j] = EX ? vsh[(size_t)t * kHeadDim + c] : (uint16_t)0;
  }

  __builtin_amdgcn_sched_barrier(0);  // keep every load above ahead of the math below

  // ---- logits: 8 threads per token, 16 channels each (correct_lane.h) -------
  {
    float ex[G], ap[G];
    if constexpr (kF2)
      run_logits<KB, G, EX, AP, false, 2>(kr, part, s_qh, s_qs, s_q4h, nullptr, s_q4c, ex, ap);
    else
      run_logits<KB, G, EX, AP, Q8, KF>(kr, part, s_qh, s_qs, s_q8h, s_q8s, s_q8c, ex, ap);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ex[h] = sum8(ex[h]);
      ap[h] = sum8(ap[h]);
    }
    if (part == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_lg[0][tl][h] = (t_sel >= 0) ? ex[h] * sm2 : -INFINITY;
        s_lg[1][tl][h] = (t_sel >= 0) ? ap[h] * sm2 : -INFINITY;
      }
    }
  }
  __syncthreads();
  if (tid < 2 * G && (EX || tid >= G) && (AP || tid < G)) {
    const int ty = tid / G, h = tid % G;
    float m = -INFINITY;
    for (int tl = 0; tl < kCorrChunk; ++tl) m = fmaxf(m, s_lg[ty][tl][h]);
    s_mx[ty][h] = m;
  }
  __syncthreads();
  {
    const int tl = tid >> 3, h = tid & 7;
    if (h < G) {
      const bool ok = s_t[tl] >= 0;
      if constexpr (EX) s_w[0][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[0][tl][h] - s_mx[0][h]) : 0.f;
      if constexpr (AP) s_w[1][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[1][tl][h] - s_mx[1][h]) : 0.f;
    }
  }
  __syncthreads();

  // ---- value sums ---------------------------------------------------------------
  float ea[G], aa[G];
#pragma unroll
  for (int h = 0; h < G; ++h) ea[h] = aa[h] = 0.f;
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    const int tl = half * kHalf + j;
    const float vx = h2f(vx16[j]);
    const float vq = AP ? vcd[j].value(max(s_t[tl], 0), c) : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (EX) ea[h] = fmaf(s_w[0][tl][h], vx, ea[h]);
      if constexpr (AP) aa[h] = fmaf(s_w[1][tl][h], vq, aa[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_part[0][half][h][c] = ea[h];
    s_part[1][half][h][c] = aa[h];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int h = e / kHeadDim, cc = e % kHeadDim;
    float* rec = cs + ((head0 + h) * nchunk + chunk) * kCsStride;
    if constexpr (EX) rec[4 + cc] = s_part[0][0][h][cc] + s_part[0][1][h][cc];
    if constexpr (AP) rec[4 + kHeadDim + cc] = s_part[1][0][h][cc] + s_part[1][1][h][cc];
  }
  if (tid < 2 * G && (EX || tid >= G) && (AP || tid < G)) {
    const int ty = tid / G, h = tid % G;
    float l = 0.f;
    for (int tl = 0; tl < kCorrChunk; ++tl) l += s_w[ty][tl][h];
    float* rec = cs + ((head0 + h) * nchunk + chunk) * kCsStride;
    rec[2 * ty] = s_mx[ty][h];
    rec[2 * ty + 1] = l;
  }
}

// Chunk terms: kBoth (exact and approximate), kExactOnly (the split states
// leave the selected tokens out), kApproxOnly (the exact state comes from
// elsewhere).
enum ChunkTerms { kBoth, kExactOnly, kApproxOnly };

template <int KB, int VB, int G, bool Q8, int KF = 0>
void launch_t(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
              const int32_t* idx, int k, const Workspace& w, ChunkTerms terms, hipStream_t s) {
  const dim3 grid(w.nchunk, L.batch * L.n_kv_heads);
  const int mshift = L.group == 64 ? 1 : 0;
  const uint8_t* kc = static_cast<const uint8_t*>(cc.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(cc.v_codes);
  if (terms == kBoth)
    chunk_kernel<KB, VB, G, true, true, Q8, KF><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, cc.k_shadow, cc.v_shadow, q,
                                                              idx, w.cs, len, L.n_q_heads, L.n_kv_heads, L.capacity,
                                                              k, w.nchunk, mshift);
  else if (terms == kExactOnly)
    chunk_kernel<KB, VB, G, true, false, false, KF><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, cc.k_shadow, cc.v_shadow,
                                                               q, idx, w.cs, len, L.n_q_heads, L.n_kv_heads,
                                                               L.capacity, k, w.nchunk, mshift);
  else
    chunk_kernel<KB, VB, G, false, true, Q8, KF><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, nullptr, nullptr, q, idx,
                                                               w.cs, len, L.n_q_heads, L.n_kv_heads, L.capacity, k,
                                                               w.nchunk, mshift);
}

template <int KB, int VB>
void launch_g(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
              const int32_t* idx, int k, const Workspace& w, ChunkTerms terms, hipStream_t s) {
  const bool q8 = L.query_bits == 8;
  if constexpr (KB == 4) {
    if (L.key_format == 1) {  // (fp16 query only)
      if (L.n_q_heads / L.n_kv_heads == 4)
        launch_t<4, VB, 4, false, 1>(L, cc, q, len, idx, k, w, terms, s);
      else
        launch_t<4, VB, 8, false, 1>(L, cc, q, len, idx, k, w, terms, s);
      return;
    }
    if (L.key_format == 2) {
      if (L.n_q_heads / L.n_kv_heads == 4)
        launch_t<4, VB, 4, false, 2>(L, cc, q, len, idx, k, w, terms, s);
      else
        launch_t<4, VB, 8, false, 2>(L, cc, q, len, idx, k, w, terms, s);
      return;
    }
  }
  if (L.n_q_heads / L.n_kv_heads == 4)
    q8 ? launch_t<KB, VB, 4, true>(L, cc, q, len, idx, k, w, terms, s)
       : launch_t<KB, VB, 4, false>(L, cc, q, len, idx, k, w, terms, s);
  else
    q8 ? launch_t<KB, VB, 8, true>(L, cc, q, len, idx, k, w, terms, s)
       : launch_t<KB, VB, 8, false>(L, cc, q, len, idx, k, w, terms, s);
}

// A second stream per device, at the default priority, with a fork and a join
// event: the block correction runs the approximate rows on it while the exact
// rows run on the caller's stream (independent parts of the same records).
// Created on the first call on a device and kept until the process ends; the
// fork-join of one call is enqueued under a lock, so calls from several host
// threads do not interleave their events.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// (under g_side_mu) The current device's side stream, or null where none can
// be made: the caller then enqueues everything on its own stream.
SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.failed) return nullptr;
  if (!ss.s) {
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      ss.failed = true;
      (void)hipGetLastError();
      return nullptr;
    }
  }
  return &ss;
}

}  // namespace

hipError_t launch_correct_rows(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                               int max_len, const int32_t* idx, int row, const Workspace& w, float* out,
                               hipStream_t s) {
  (void)hipGetLastError();  // report only this call's launches
  // records per query head: at most w.nchunk (records of kCorrChunk entries over min(row, max_len))
  const int nrec = (min(row, max_len) + kRowRec - 1) / kRowRec;
  if (nrec > 0) {
    const dim3 grid(nrec, L.batch * L.n_kv_heads);
    // the approximate rows on the side stream, forked from and joined back
    // into the caller's stream around the exact rows
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* ss = side_stream();
    hipStream_t sa = s;
    if (ss && hipEventRecord(ss->fork, s) == hipSuccess && hipStreamWaitEvent(ss->s, ss->fork, 0) == hipSuccess)
      sa = ss->s;
    const hipError_t ea = launch_rows_approx(L, c, q, len, w, idx, row, nrec, sa);
    if (ea != hipSuccess) return ea;
    if (sa != s && hipEventRecord(ss->join, sa) != hipSuccess) return hipErrorLaunchFailure;
    if (L.n_q_heads / L.n_kv_heads == 4)
      exact_rows_kernel<4><<<grid, 64 * kRowWaves, 0, s>>>(c.k_shadow, c.v_shadow, q, idx, w.cs, len, L.n_q_heads,
                                                          L.n_kv_heads, L.capacity, row, w.nchunk);
    else
      exact_rows_kernel<8><<<grid, 64 * kRowWaves, 0, s>>>(c.k_shadow, c.v_shadow, q, idx, w.cs, len, L.n_q_heads,
                                                          L.n_kv_heads, L.capacity, row, w.nchunk);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    // the combine after both parts
    if (sa != s && hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return hipErrorLaunchFailure;
  }
  if (nrec <= 8 && w.nsplit <= 8)
    combine_kernel<1, 8><<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, nullptr,
                                                                        out, len, L.n_q_heads, w.nsplit, w.nchunk,
                                                                        row, 0, kRowRec);
  else if (nrec <= kRecBatchMax && w.nsplit <= kRecBatchMax)
    combine_kernel<1><<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, nullptr,
                                                                     out, len, L.n_q_heads, w.nsplit, w.nchunk, row,
                                                                     0, kRowRec);
  else
    combine_kernel<4><<<dim3(L.n_q_heads, L.batch), kHeadDim * 4, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs,
                                                                         nullptr, out, len, L.n_q_heads, w.nsplit,
                                                                         w.nchunk, row, 0, kRowRec);
  return hipGetLastError();
}

hipError_t launch_correct(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                          const SeqArg& len, const int32_t* idx, int k, const Workspace& w,
                          const float* hx, bool rest, float* out, hipStream_t s) {
  (void)hipGetLastError();  // report only this call's launches
  const ChunkTerms t = hx ? kApproxOnly : (rest ? kExactOnly : kBoth);
  if (w.nchunk > 0) {
    const bool v4 = L.v_bits == 4;
    switch (L.k_bits) {
      case 4: v4 ? launch_g<4, 4>(L, c, q, len, idx, k, w, t, s) : launch_g<4, 2>(L, c, q, len, idx, k, w, t, s); break;
      case 3: v4 ? launch_g<3, 4>(L, c, q, len, idx, k, w, t, s) : launch_g<3, 2>(L, c, q, len, idx, k, w, t, s); break;
      case 2: v4 ? launch_g<2, 4>(L, c, q, len, idx, k, w, t, s) : launch_g<2, 2>(L, c, q, len, idx, k, w, t, s); break;
      default: v4 ? launch_g<1, 4>(L, c, q, len, idx, k, w, t, s) : launch_g<1, 2>(L, c, q, len, idx, k, w, t, s);
    }
  }
  if (w.nchunk <= 8 && w.nsplit <= 8)  // every record list fits one batch of 8
    combine_kernel<1, 8><<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, hx, out,
                                                                        len, L.n_q_heads, w.nsplit, w.nchunk, k,
                                                                        rest ? 1 : 0, kCorrChunk);
  else if (w.nchunk <= kRecBatchMax && w.nsplit <= kRecBatchMax)  // every record list fits one batch
    combine_kernel<1><<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, hx, out,
                                                                     len, L.n_q_heads, w.nsplit, w.nchunk, k,
                                                                     rest ? 1 : 0, kCorrChunk);
  else
    combine_kernel<4><<<dim3(L.n_q_heads, L.batch), kHeadDim * 4, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, hx,
                                                                         out, len, L.n_q_heads, w.nsplit, w.nchunk,
                                                                         k, rest ? 1 : 0, kCorrChunk);
  return hipGetLastError();
}

}  // namespace bkv
