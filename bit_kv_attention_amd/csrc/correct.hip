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
#include "bkv_internal.h"
#include "quant_lane.h"

namespace bkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

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
                                                           int rest) {
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
  const int nc = (kk + kCorrChunk - 1) / kCorrChunk;
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

// EX = false: only the approximate terms (the exact state comes from
// elsewhere, see qattn_correct_hybrid); the shadow rows are not read.
// AP = false: only the exact terms (the approximate state already leaves the
// selected tokens out, see qattn_decode_unselected); the packed cache is not
// read.
// Q8: the approximate logits take the INT8 query of the scan (quant_lane.h).
// MX: the key codes are MXFP4 (E2M1 numbers, one power-of-two scale per group
// of 32, no zero point).
template <int KB, int VB, int G, bool EX, bool AP = true, bool Q8 = false, bool MX = false>
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
    }
    if (tid < kCorrChunk) s_t[tid] = (ii < kk && tv >= 0 && tv < n) ? tv : -1;
  }
  __syncthreads();

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  const uint32_t* kmeta = k_meta + (size_t)u * meta_planes(mshift) * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * meta_planes(mshift) * cap;
  const uint16_t* ksh = k_shadow + (size_t)u * cap * kHeadDim;
  const uint16_t* vsh = v_shadow + (size_t)u * cap * kHeadDim;

  // ---- loads: the keys of the logits, then the values; all unconditional (an
  // empty slot reads token 0, always present when a chunk runs, and is masked
  // later) so that every load is in flight before the first is needed -------
  const int tl = tid >> 3;
  const int part = tid & 7;
  const int t_sel = s_t[tl];
  const int c0 = 16 * part;
  uint4 k0, k1;
  uint32_t kraw[2][2];
  uint32_t kmw;
  {
    const int t = max(t_sel, 0);
    if constexpr (EX) {
      const uint4* kr = reinterpret_cast<const uint4*>(ksh + (size_t)t * kHeadDim + c0);
      k0 = kr[0];
      k1 = kr[1];
    } else {
      k0 = k1 = (uint4){0u, 0u, 0u, 0u};
    }
    // channels c0..c0+15 are the group-(part/2) fields of the chunks of
    // eighths 2*(part%2) and 2*(part%2)+1 (8*KB bits each)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t* ch = reinterpret_cast<const uint32_t*>(kbase + k_chunk_offset(KB, t, 2 * (part & 1) + x));
      const int d0 = (8 * KB * (part >> 1)) >> 5, d1 = min(d0 + 1, KB - 1);
      kraw[x][0] = AP ? ch[d0] : 0u;
      kraw[x][1] = AP ? ch[d1] : 0u;
    }
    kmw = AP ? kmeta[(size_t)((c0 / kGroup) >> mshift) * cap + t] : 0u;
  }
  // value loads: one thread per (channel, half of the chunk)
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  constexpr int kHalf = kCorrChunk / 2;
  uint16_t vx16[kHalf];
  uint32_t vcode[kHalf], vmw[kHalf];
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    const int t = max(s_t[half * kHalf + j], 0);
    int dw, bit;
    v_code_pos(VB, t % kTile, c, dw, bit);
    const uint32_t* vt = reinterpret_cast<const uint32_t*>(vbase + (size_t)(t / kTile) * v_tile_bytes(VB));
    vcode[j] = AP ? vt[dw] : 0u;  // raw: shifted at use, after the loads have landed
    vmw[j] = AP ? vmeta[(size_t)((c / kGroup) >> mshift) * cap + t] : 0u;
    vx16[j] = EX ? vsh[(size_t)t * kHeadDim + c] : (uint16_t)0;
  }

  __builtin_amdgcn_sched_barrier(0);  // keep every load above ahead of the math below

  // ---- logits: 8 threads per token, 16 channels each ------------------------
  // fp16 pairs through v_dot2_f32_f16 (exact products, fp32 sums): the exact
  // key pairs, and for the approximate logit the codes as exact fp16
  // integers, whose dot product with q takes the group's scale once, plus
  // zero x (sum of q over the run) -- the scan's own form of the score.
  {
    float ex[G], ap[G];
    {
      const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const int sh = (8 * KB * (part >> 1)) & 31;
      uint32_t fld[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) fld[x] = (uint32_t)((((uint64_t)kraw[x][1] << 32) | kraw[x][0]) >> sh);
      const uint64_t bits = ((uint64_t)fld[0] & ((1ull << (8 * KB)) - 1)) | ((uint64_t)fld[1] << (8 * KB));
      constexpr uint32_t M = (1u << KB) - 1;
      const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
      half2_t cp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (uint32_t)(bits >> (KB * 2 * i)) & M, hi = (uint32_t)(bits >> (KB * (2 * i + 1))) & M;
        if constexpr (MX)  // the fp16 pattern of the E2M1 value * 2^-14 (exact)
          cp[i] = __builtin_bit_cast(half2_t, ((lo & 7u) << 9) | ((lo & 8u) << 12) | ((hi & 7u) << 25) | ((hi & 8u) << 28));
        else
          cp[i] = __builtin_bit_cast(half2_t, lo | (hi << 16) | 0x64006400u) - k1024;
      }
      const float s = h2f((uint16_t)(kmw & 0xFFFFu)) * (MX ? 16384.0f : 1.0f), z = h2f((uint16_t)(kmw >> 16));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 qa = s_qh[h][2 * part], qb = s_qh[h][2 * part + 1];
        const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        uint32_t qw8[8];
        if constexpr (Q8) {  // q' as exact fp16 integers: q' . code is an exact integer sum
          const uint4 ra = s_q8h[h][2 * part], rb = s_q8h[h][2 * part + 1];
          const uint32_t r8[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) qw8[i] = r8[i];
        }
        float e = 0.f, d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const half2_t qq = __builtin_bit_cast(half2_t, qw[i]);
          if constexpr (EX) e = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kw[i]), qq, e, false);
          if constexpr (AP) d = __builtin_amdgcn_fdot2(cp[i], Q8 ? __builtin_bit_cast(half2_t, qw8[i]) : qq, d, false);
        }
        ex[h] = e;
        if constexpr (Q8)
          ap[h] = AP ? fmaf(s, d * s_q8c[h][part], z * s_q8s[h][part]) : 0.f;
        else
          ap[h] = AP ? fmaf(s, d, z * s_qs[h][part]) : 0.f;
      }
    }
    // sum over the token's 8 threads (lanes 8m..8m+7): quads by DPP, then the
    // other quad (row_ror:12 brings lane l+4 to lanes 0 and 8 of each row)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ex[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ex[h]), 0xB1, 0xF, 0xF, true));
      ap[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ap[h]), 0xB1, 0xF, 0xF, true));
      ex[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ex[h]), 0x4E, 0xF, 0xF, true));
      ap[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ap[h]), 0x4E, 0xF, 0xF, true));
      ex[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ex[h]), 0x12C, 0xF, 0xF, true));
      ap[h] += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ap[h]), 0x12C, 0xF, 0xF, true));
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
    int dw, bit;
    v_code_pos(VB, max(s_t[tl], 0) % kTile, c, dw, bit);
    const float vq = fmaf(h2f((uint16_t)(vmw[j] & 0xFFFFu)), (float)((vcode[j] >> bit) & ((1u << VB) - 1)),
                          h2f((uint16_t)(vmw[j] >> 16)));
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

template <int KB, int VB, int G, bool Q8, bool MX = false>
void launch_t(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
              const int32_t* idx, int k, const Workspace& w, ChunkTerms terms, hipStream_t s) {
  const dim3 grid(w.nchunk, L.batch * L.n_kv_heads);
  const int mshift = L.group == 64 ? 1 : 0;
  const uint8_t* kc = static_cast<const uint8_t*>(cc.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(cc.v_codes);
  if (terms == kBoth)
    chunk_kernel<KB, VB, G, true, true, Q8, MX><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, cc.k_shadow, cc.v_shadow, q,
                                                              idx, w.cs, len, L.n_q_heads, L.n_kv_heads, L.capacity,
                                                              k, w.nchunk, mshift);
  else if (terms == kExactOnly)
    chunk_kernel<KB, VB, G, true, false><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, cc.k_shadow, cc.v_shadow,
                                                               q, idx, w.cs, len, L.n_q_heads, L.n_kv_heads,
                                                               L.capacity, k, w.nchunk, mshift);
  else
    chunk_kernel<KB, VB, G, false, true, Q8, MX><<<grid, 256, 0, s>>>(kc, vc, cc.k_meta, cc.v_meta, nullptr, nullptr, q, idx,
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
        launch_t<4, VB, 4, false, true>(L, cc, q, len, idx, k, w, terms, s);
      else
        launch_t<4, VB, 8, false, true>(L, cc, q, len, idx, k, w, terms, s);
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

}  // namespace

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
                                                                        rest ? 1 : 0);
  else if (w.nchunk <= kRecBatchMax && w.nsplit <= kRecBatchMax)  // every record list fits one batch
    combine_kernel<1><<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, hx, out,
                                                                     len, L.n_q_heads, w.nsplit, w.nchunk, k,
                                                                     rest ? 1 : 0);
  else
    combine_kernel<4><<<dim3(L.n_q_heads, L.batch), kHeadDim * 4, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, hx,
                                                                         out, len, L.n_q_heads, w.nsplit, w.nchunk,
                                                                         k, rest ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bkv
