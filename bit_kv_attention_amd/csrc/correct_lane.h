// correct_lane.h -- the per-thread pieces of the exact correction, shared by
// the correction kernel (correct.hip) and the fused step's tail
// (decode_approx.hip): the loads of one selected token's 16-channel key run
// and of its value codes, and the exact and approximate logits of that run.
//
// A selected token's logits are split over 8 threads, thread `part` taking
// channels 16*part .. 16*part + 15; the caller sums the 8 partial logits.
//   exact:        q . k over the run, k the fp16 shadow row (JetFire README,
//                 introduction: the top-k tokens are corrected with exact
//                 high-precision keys and values);
//   approximate:  s * (q . code) + z * (sum of q over the run), with the
//                 codes as exact fp16 integers -- the scan's own form of the
//                 score (HACK review on Pith, Eq. (4), unquantised query);
//                 INT8 query: s_q * s * (q' . code) + z * s_q * (sum q');
//                 MXFP4 keys: s * (q . e2m1(code)), no zero point;
//                 MXFP4 keys and query (key format 2): 2^(Xq + Xk) *
//                 (e2m1(q) . e2m1(code)) for the run's quarter, the query
//                 quantised by quantise_lane_e8 like the keys (the scan's
//                 FP4 product, Jet-QSparse abstract).
// Products are exact in v_dot2_f32_f16 (fp16 pairs, fp32 sums).  With E2M1
// operands on both sides every product and every partial sum is exact, so a
// run's FP4 logit is exact before the sum over the 8 threads.
#pragma once

#include "bkv_internal.h"

namespace bkv {

typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));

__device__ inline float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// The raw loads of channels 16*part .. 16*part + 15 of token t.  Channels
// c0..c0+15 are the group-(part/2) fields of the key chunks of eighths
// 2*(part%2) and 2*(part%2)+1 (8*KB bits each); in key format 2 (KF = 2) they
// are bytes 8*(part%2) .. +7 of the token's chunk of quarter part/2, and the
// meta word is the token's word of four E8M0 scale bytes.  EX: the shadow row
// is read; AP: the codes and the meta word are read.
template <int KB, bool EX, bool AP, int KF = 0>
struct KeyRun {
  uint4 k0, k1;         // fp16 shadow channels c0..c0+7, c0+8..c0+15
  uint32_t kraw[2][2];  // the two key chunks' dwords holding the run's fields
  uint32_t kmw;         // meta word of the run's group (fp16 scale low, zero high)

  __device__ inline void load(const uint16_t* __restrict__ ksh, const uint8_t* __restrict__ kbase,
                              const uint32_t* __restrict__ kmeta, int cap, int t, int part, int mshift) {
    const int c0 = 16 * part;
    if constexpr (EX) {
      const uint4* kr = reinterpret_cast<const uint4*>(ksh + (size_t)t * kHeadDim + c0);
      k0 = kr[0];
      k1 = kr[1];
    } else {
      k0 = k1 = (uint4){0u, 0u, 0u, 0u};
    }
    if constexpr (KF == 2) {  // (kmeta: the unit's plane of scale words)
      const uint2 w = AP ? *reinterpret_cast<const uint2*>(kbase + k_chunk_offset_e8(t, part >> 1) + 8 * (part & 1))
                         : (uint2){0u, 0u};
      kraw[0][0] = w.x;
      kraw[0][1] = w.y;
      kraw[1][0] = kraw[1][1] = 0u;
      kmw = AP ? kmeta[t] : 0u;
      return;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t* ch = reinterpret_cast<const uint32_t*>(kbase + k_chunk_offset(KB, t, 2 * (part & 1) + x));
      const int d0 = (8 * KB * (part >> 1)) >> 5, d1 = min(d0 + 1, KB - 1);
      kraw[x][0] = AP ? ch[d0] : 0u;
      kraw[x][1] = AP ? ch[d1] : 0u;
    }
    kmw = AP ? kmeta[(size_t)((c0 / kGroup) >> mshift) * cap + t] : 0u;
  }

  // The run's 16 codes as 8 fp16 pairs (channel pairs in order): exact
  // integers (affine codes) or the fp16 pattern of the E2M1 value * 2^-14
  // (MXFP4: magnitude bits into the exponent's low bits and the mantissa's
  // top bit, the sign bit into fp16's sign).
  template <bool MX>
  __device__ inline void codes(int part, half2v_t (&cp)[8]) const {
    uint64_t bits;
    if constexpr (KF == 2) {  // 16 codes in channel order, 4 bits each
      bits = ((uint64_t)kraw[0][1] << 32) | kraw[0][0];
    } else {
      const int sh = (8 * KB * (part >> 1)) & 31;
      uint32_t fld[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) fld[x] = (uint32_t)((((uint64_t)kraw[x][1] << 32) | kraw[x][0]) >> sh);
      bits = ((uint64_t)fld[0] & ((1ull << (8 * KB)) - 1)) | ((uint64_t)fld[1] << (8 * KB));
    }
    constexpr uint32_t M = (1u << KB) - 1;
    const half2v_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (uint32_t)(bits >> (KB * 2 * i)) & M, hi = (uint32_t)(bits >> (KB * (2 * i + 1))) & M;
      if constexpr (MX)
        cp[i] = __builtin_bit_cast(half2v_t, ((lo & 7u) << 9) | ((lo & 8u) << 12) | ((hi & 7u) << 25) | ((hi & 8u) << 28));
      else
        cp[i] = __builtin_bit_cast(half2v_t, lo | (hi << 16) | 0x64006400u) - k1024;
    }
  }
};

// Exact and approximate partial logits (not yet scaled by 1/sqrt(D)) of the
// run for the G query heads.  qh: the query rows as fp16 pairs [G][16];
// qs: sums of q over 16-channel runs [G][8].  Q8: q8h = the INT8 codes q' as
// fp16 pairs, q8s = s_q * (sum of q' over the run), q8c = s_q of the run's
// group.  KF (key format) 1: MXFP4 keys against the fp16 query; 2: MXFP4 keys
// against the MXFP4 query, q8h = the query's E2M1 codes as the fp16 patterns
// of their values * 2^-14 and q8c = 2^(Xq + 28) of the run's quarter (the
// two 2^-14 undone), q8s unused.
template <int KB, int G, bool EX, bool AP, bool Q8, int KF>
__device__ inline void run_logits(const KeyRun<KB, EX, AP, KF>& r, int part, const uint4 (*qh)[kHeadDim / 8],
                                  const float (*qs)[kHeadDim / 16], const uint4 (*q8h)[kHeadDim / 8],
                                  const float (*q8s)[kHeadDim / 16], const float (*q8c)[kHeadDim / 16],
                                  float (&ex)[G], float (&ap)[G]) {
  const uint32_t kw[8] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w, r.k1.x, r.k1.y, r.k1.z, r.k1.w};
  constexpr bool MX = KF != 0;
  constexpr bool QC = Q8 || KF == 2;  // the approximate logits take the quantised query q8h
  half2v_t cp[8];
  r.template codes<MX>(part, cp);
  const float s = h2f((uint16_t)(r.kmw & 0xFFFFu)) * (MX ? 16384.0f : 1.0f), z = h2f((uint16_t)(r.kmw >> 16));
  // key format 2: 2^(Xk) from the quarter's E8M0 byte (101..140: a normal float)
  const float ks = __uint_as_float(((r.kmw >> (8 * (part >> 1))) & 0xFFu) << 23);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qa = qh[h][2 * part], qb = qh[h][2 * part + 1];
    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    uint32_t qw8[8];
    if constexpr (QC) {  // q' as exact fp16 integers (or FP4 patterns): an exact sum
      const uint4 ra = q8h[h][2 * part], rb = q8h[h][2 * part + 1];
      const uint32_t r8[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) qw8[i] = r8[i];
    }
    float e = 0.f, d = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const half2v_t qq = __builtin_bit_cast(half2v_t, qw[i]);
      if constexpr (EX) e = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v_t, kw[i]), qq, e, false);
      if constexpr (AP) d = __builtin_amdgcn_fdot2(cp[i], QC ? __builtin_bit_cast(half2v_t, qw8[i]) : qq, d, false);
    }
    ex[h] = e;
    if constexpr (KF == 2)
      ap[h] = AP ? (d * q8c[h][part]) * ks : 0.f;
    else if constexpr (Q8)
      ap[h] = AP ? fmaf(s, d * q8c[h][part], z * q8s[h][part]) : 0.f;
    else
      ap[h] = AP ? fmaf(s, d, z * qs[h][part]) : 0.f;
  }
}

// Sum over the token's 8 threads (lanes 8m..8m+7 of a wave): quads by DPP,
// then the other quad (row_ror:12 brings lane l+4 to lanes 0 and 8 of each
// row of 16).  Lane 8m holds the total.
__device__ inline float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x12C, 0xF, 0xF, true));
  return x;
}

// One value code of (token t, channel c): the raw dword holding it and the
// group's meta word; value() shifts it out after the loads have landed.
template <int VB>
struct ValueCode {
  uint32_t dw, mw;
  __device__ inline void load(const uint8_t* __restrict__ vbase, const uint32_t* __restrict__ vmeta, int cap, int t,
                              int c, int mshift) {
    int d, bit;
    v_code_pos(VB, t % kTile, c, d, bit);
    dw = reinterpret_cast<const uint32_t*>(vbase + (size_t)(t / kTile) * v_tile_bytes(VB))[d];
    mw = vmeta[(size_t)((c / kGroup) >> mshift) * cap + t];
  }
  __device__ inline float value(int t, int c) const {  // s * code + z
    int d, bit;
    v_code_pos(VB, t % kTile, c, d, bit);
    return fmaf(h2f((uint16_t)(mw & 0xFFFFu)), (float)((dw >> bit) & ((1u << VB) - 1)), h2f((uint16_t)(mw >> 16)));
  }
};

}  // namespace bkv
