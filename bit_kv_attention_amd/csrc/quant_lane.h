// quant_lane.h -- the per-group quantiser of appended tokens, shared by the
// append kernel and the scan's in-launch append (both must produce the same
// bits).
//
// Per token, per K/V, per group (the asymmetric per-group quantiser of the
// HACK review on Pith, Eq. (4): zero point = group minimum, step = range /
// (2^b - 1); fp16 zero point and scale as in the TailorKV review's
// free-parameter list):
//   z = min x,  s = fp16((max - min) / (2^b - 1))   [fp32 subtract, IEEE divide]
//   code = clamp(rint((x - z) / s), 0, 2^b - 1)     [stored fp16 s and z; 0 if s == 0]
//
// Four lanes share one 32-channel quarter of a row (8 channels each; lane
// sub = l & 3, quarter grp = (l >> 2) & 3 of a 16-lane set): partial min/max
// per lane, merged across the four lanes (and, for groups of 64, with the
// quarter pair's lanes l ^ 4) with ties resolved toward the lower channels,
// so the result -- including the sign of a zero minimum -- is that of one
// sequential pass in channel order.  Every lane of the set must be active.
#pragma once

#include "bkv_internal.h"

namespace bkv {

// x: this lane's 8 values; returns the group's meta word (fp16 scale low,
// fp16 zero high) and the lane's 8 codes.
__device__ inline uint32_t quantise_lane(const float (&x)[8], int sub, int grp, int mshift, float qmax,
                                         uint32_t (&code)[8]) {
#pragma clang fp contract(off)
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (x[j] < mn) mn = x[j];
    if (x[j] > mx) mx = x[j];
  }
  auto merge = [&](float omn, float omx, bool hi) {  // hi: the partner holds the lower channels
    const float lmn = hi ? omn : mn, umn = hi ? mn : omn;
    const float lmx = hi ? omx : mx, umx = hi ? mx : omx;
    mn = (umn < lmn) ? umn : lmn;
    mx = (umx > lmx) ? umx : lmx;
  };
  merge(__int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0xB1, 0xF, 0xF, true)),
        __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0xB1, 0xF, 0xF, true)), (sub & 1) != 0);
  merge(__int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x4E, 0xF, 0xF, true)),
        __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xF, 0xF, true)), (sub & 2) != 0);
  if (mshift)  // group 64: the quarter pair's lanes (l ^ 4) hold the group's other half
    merge(__shfl_xor(mn, 4), __shfl_xor(mx, 4), (grp & 1) != 0);
  const _Float16 s16 = (_Float16)((mx - mn) / qmax);
  const _Float16 z16 = (_Float16)mn;
  const float s = (float)s16, z = (float)z16;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int cd = 0;
    if (s != 0.0f) {
      const float rr = __builtin_rintf((x[j] - z) / s);
      cd = rr < 0.0f ? 0 : (rr > qmax ? (int)qmax : (int)rr);
    }
    code[j] = (uint32_t)cd;
  }
  return (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
}

// MXFP4 keys (Jet-QSparse abstract: FP4 keys; the OCP Microscaling block
// format): the 32 channels of a quarter share the scale 2^X with
// X = floor(log2(amax)) - 2, clamped at -24 so that it is an fp16 value;
// each code is sign << 3 | the E2M1 magnitude index of |x| / 2^X, rounded to
// nearest with ties to the even index and clamped at 6.  Meta word: fp16 2^X
// low, 0 high (0 for an all-zero quarter).  Same lane set as quantise_lane
// (a quad per quarter, groups of 32 only).
__device__ inline uint32_t quantise_lane_mx(const float (&x)[8], uint32_t (&code)[8]) {
#pragma clang fp contract(off)
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  if (a == 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) code[j] = 0u;
    return 0u;
  }
  // a >= 2^-24 is a normal fp32 number: its exponent field is floor(log2 a)
  const int X = max((int)((__float_as_uint(a) >> 23) & 0xFFu) - 127 - 2, -24);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = __builtin_amdgcn_ldexpf(fabsf(x[j]), -X);  // exact
    const int idx = (r > 0.25f) + (r >= 0.75f) + (r > 1.25f) + (r >= 1.75f) + (r > 2.5f) + (r >= 3.5f) + (r > 5.0f);
    code[j] = (uint32_t)(idx | ((x[j] < 0.0f && idx != 0) ? 8 : 0));
  }
  const uint32_t s16 = (X >= -14) ? (uint32_t)(X + 15) << 10 : 1u << (X + 24);
  return s16;
}

// Key format 2 and its query (OCP Microscaling block format with the scale
// kept as E8M0; the Jet-QSparse abstract's FP4 query-key product): the same
// rounding as quantise_lane_mx, but X = floor(log2(amax)) - 2 is not clamped
// (fp16 inputs put it in [-26, 13]) and the result is the E8M0 byte X + 127
// (127 for an all-zero quarter, whose codes are all 0).  Same lane set.
__device__ inline uint32_t quantise_lane_e8(const float (&x)[8], uint32_t (&code)[8]) {
#pragma clang fp contract(off)
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  if (a == 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) code[j] = 0u;
    return 127u;
  }
  // a >= 2^-24 is a normal fp32 number: its exponent field is floor(log2 a)
  const int X = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127 - 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = __builtin_amdgcn_ldexpf(fabsf(x[j]), -X);  // exact
    const int idx = (r > 0.25f) + (r >= 0.75f) + (r > 1.25f) + (r >= 1.75f) + (r > 2.5f) + (r >= 3.5f) + (r > 5.0f);
    code[j] = (uint32_t)(idx | ((x[j] < 0.0f && idx != 0) ? 8 : 0));
  }
  return (uint32_t)(X + 127);
}

// The 8 codes of a lane (channels 32grp + 8sub + j) into their key chunk of
// key format 2: nibbles 8sub .. 8sub+7, i.e. the chunk's dword sub.
__device__ inline void store_key_codes_e8(uint8_t* __restrict__ unit_codes, int t, int sub, int grp,
                                          const uint32_t (&code)[8]) {
  uint32_t f = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) f |= code[j] << (4 * j);
  *reinterpret_cast<uint32_t*>(unit_codes + k_chunk_offset_e8(t, grp) + 4 * sub) = f;
}

// The 8 fp16 values of a 16-byte piece as floats (exact).
__device__ inline void halves8(const uint4& w4, float (&x)[8]) {
  const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ww[j] & 0xFFFFu));
    x[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(ww[j] >> 16));
  }
}

// The 8 codes of a lane into its key chunk: chunk (eighth sub) of token t
// holds codes (g, j) at bit KB(8g + j), so quarter grp's 8 codes fill bytes
// KB*grp .. KB*grp + KB - 1.
template <int KB>
__device__ inline void store_key_codes(uint8_t* __restrict__ unit_codes, int t, int sub, int grp,
                                       const uint32_t (&code)[8]) {
  uint32_t f = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) f |= code[j] << (KB * j);
  uint8_t* chunk = unit_codes + k_chunk_offset(KB, t, sub) + KB * grp;
  if (KB == 4) {
    *reinterpret_cast<uint32_t*>(chunk) = f;
  } else {
#pragma unroll
    for (int i = 0; i < KB; ++i) chunk[i] = (uint8_t)(f >> (8 * i));
  }
}

// ---- the INT8 query of the approximate scores -------------------------------
// (HACK review on Pith, Eq. (4): both operands of Q.K^T quantised per
// partition, the product formed on the integer codes.)  The query's partition
// is the layout's group and is symmetric: s = amax / 127 in fp32 (correctly
// rounded divide), q' = rint(q / s) in [-127, 127], 0 when s == 0.  With a
// zero point of 0, Eq. (4) for a key group s_k*k' + z_k keeps two terms:
//   q_hat . k_hat = s * (s_k * (q' . k') + z_k * sum(q')).
// The scan and the correction both quantise with these two functions, so
// their codes agree bit for bit.
__device__ inline float query_scale_i8(float amax) {
#pragma clang fp contract(off)
  return amax / 127.0f;
}
__device__ inline int query_code_i8(float x, float s) {
#pragma clang fp contract(off)
  if (s == 0.0f) return 0;
  const float r = __builtin_rintf(x / s);
  return (int)fminf(fmaxf(r, -127.0f), 127.0f);
}

}  // namespace bkv
