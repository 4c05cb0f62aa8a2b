// decode_approx.hip -- the approximate pass over the packed low-bit cache.
//
// What it computes (JetFire README, introduction: attention over the low-bit
// cache is the "approximate" half of approximate-then-correct):
//   s_hat[h][t] = (1/sqrt(D)) * sum_g ( s_g,t * (q_h,g . code_g,t) + z_g,t * sum(q_h,g) )
// which is q_h . (s*code + z) rearranged as in the HACK review's Eq. (4) with an
// unquantised query, so the codes enter the contraction as exact small
// integers; sigma[t] = max over the KV head's query heads of s_hat; and, per
// split of the token range, the online-softmax state of sum_t p_t * V_hat_t
// with V_hat = s*code + z applied the same way (sum p*s*code + sum p*z).
//
// Mapping onto gfx950 (one workgroup = kScanWaves waves = one (b, kvh) unit and one
// split; each wave takes 32-token steps):
//  * Scores: v_mfma_f32_16x16x32_f16 with A = 16 tokens x the 32 codes of one
//    quantisation group (exact integers in fp16) and B = 16 columns that pair
//    (group g', query head h).  Column (g', h) carries q_h's group-g' channels
//    at K-step g' and zeros at the other K-steps, so after the four K-steps
//    D[t][(g',h)] = q_h,g' . code_g',t: the per-(token, group) scale is applied
//    once per output element and the GQA group fills the otherwise padded N.
//    (G = 8 needs 32 columns: two N-tiles, groups {0,1} and {2,3}.)
//  * The D layout leaves, in each lane, head h's logits for tokens
//    {4kb..4kb+3} and {16+4kb..16+4kb+3} of the step (kb = lane/16).  That is
//    exactly the K-slot set the P.V MFMA wants in the same lane when its A
//    operand is the token-tiled V word (channel, kb) -- the V layout is chosen
//    so, and no cross-lane shuffle is needed between the two contractions.
//  * P.V: v_mfma_f32_16x16x32_f16 with A = 16 channels x 32 tokens of V codes
//    and B = columns (g, h) holding fp16(p * s_g,t); channel tile nt only keeps
//    the columns of its own group.  sum p*z is accumulated on the VALU.
//  * Key codes become exact fp16 integers (OR into 1024 + c, subtract 1024);
//    pairs 1 and 3 are masked in place at bit KB, i.e. as 2^KB * c, and the
//    query operand carries 2^-KB on those slots (one shift per two pairs).
//    Value codes enter as fp16 subnormals (the masked bit pattern c is the
//    value c * 2^-24), one shift and one AND per pair, no conversion.
//  * Memory: the packed layouts put each lane's operands at byte 16*lane (key
//    chunks: 12*lane for 3 bits) of contiguous 1 KB runs, so a wave's step is
//    4-6 fully coalesced 16-byte-per-lane loads, prefetched one step ahead
//    into a second register set.  The scale/zero words, which several lanes
//    share, are loaded once (one 16-byte load per lane covers the step's K
//    and V meta) and handed out through a per-wave LDS slot.  Selection scores
//    are staged in LDS and stored every 8 steps as one coalesced store.
//
// INT8 query (HACK review on Pith, Eq. (4), both operands of Q.K^T quantised):
// this file is built a second time with BKV_QUERY_INT8=1.  That build
// quantises each query group to symmetric INT8 codes q' with an fp32 scale s
// (quant_lane.h), takes the scores on v_mfma_i32_16x16x32_i8 with A = the
// key codes as bytes and B = q' (exact integer sums), and applies s with the
// key group's scale: s_hat = sum_g s_k * (s * (q' . k')) + z_k * (s * sum q').
// Key codes become bytes with two or three VALU operations per 8 codes (no
// fp16 conversion); a lane's 8 bytes take the channels in the order
// key_byte_channel gives, and the query operand follows the same order.
//
// MXFP4 keys (Jet-QSparse abstract: FP4 keys; OCP Microscaling block format):
// a third build, BKV_KEY_MXFP4=1, for 4-bit keys whose codes are E2M1
// numbers with one power-of-two scale per group of 32 (quant_lane.h).  An
// E2M1 code becomes an exact fp16 operand with three VALU operations per two
// codes (unpack_keys_mx: its bits are the fp16 pattern of value * 2^-14), the
// scores run on the same fp16 MFMA with the group's scale applied after it,
// and the 2^14 is folded into the constants that turn scores into sigma and
// log2 units.
//
// MXFP4 keys and query (key format 2; Jet-QSparse abstract: FP4 keys with a
// native FP4 query-key product): a fourth build, BKV_KEY_FP4=1.  Each
// workgroup quantises its G query rows per 32-channel quarter to E2M1 codes
// with an E8M0 scale (quantise_lane_e8, the keys' own rule), and a 16-token
// tile's scores are one v_mfma_scale_f32_16x16x128_f8f6f4: A = the tile's
// 1 KB of key chunks as loaded (lane (kb, n) holds quarter kb of token n, see
// k_chunk_offset_e8) with the token's E8M0 byte of that quarter as its
// scale; B = column n holding query head n mod G (the GQA group repeated
// across the 16 columns) with that head's quarter scale.  Both scales are
// applied inside the MFMA, so each output element is already the whole
// logit, in the same lane positions the fp16 path reaches after its
// reduction over groups; no key is unpacked on the VALU.  The key scale
// words (one per token) travel through the per-wave meta slot like the
// other meta.
#include "bkv_internal.h"
#include "fused_tail.h"
#include "quant_lane.h"
#include "select_lds.h"

#ifndef BKV_QUERY_INT8
#define BKV_QUERY_INT8 0
#endif
#ifndef BKV_KEY_MXFP4
#define BKV_KEY_MXFP4 0
#endif
#ifndef BKV_KEY_FP4
#define BKV_KEY_FP4 0
#endif
#if BKV_QUERY_INT8
#define BKV_SCAN_KERNEL decode_approx_q8_kernel
#define BKV_SCAN_LAUNCH launch_decode_approx_q8
#define BKV_ROWS_LAUNCH launch_rows_approx_q8
#elif BKV_KEY_MXFP4
#define BKV_SCAN_KERNEL decode_approx_mx_kernel
#define BKV_SCAN_LAUNCH launch_decode_approx_mx
#define BKV_ROWS_LAUNCH launch_rows_approx_mx
#elif BKV_KEY_FP4
#define BKV_SCAN_KERNEL decode_approx_fp4_kernel
#define BKV_SCAN_LAUNCH launch_decode_approx_fp4
#define BKV_ROWS_LAUNCH launch_rows_approx_fp4
#else
#define BKV_SCAN_KERNEL decode_approx_kernel
#define BKV_SCAN_LAUNCH launch_decode_approx
#define BKV_ROWS_LAUNCH launch_rows_approx
#endif

namespace bkv {
namespace {

constexpr bool kQ8 = BKV_QUERY_INT8 != 0;
constexpr bool kMX = BKV_KEY_MXFP4 != 0;
constexpr bool kFP4 = BKV_KEY_FP4 != 0;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// DPP helpers (row = 16 lanes).
// The patterns used (quad_perm, row_ror) read a valid lane for every lane, so
// `old` is irrelevant; leaving it undefined lets the compiler fold the move
// into the consuming add/max.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Max with the lane 16 (32) apart, by the gfx950 row swaps: with both operands
// x, permlane16_swap returns (x of the even row of each row pair in both, x of
// the odd row in both) -- i.e. own and partner values in some order (likewise
// for the halves with permlane32_swap); no LDS round trip.
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// y holds 4 codes of `BITS` bits in its low half and 4 in its high half (code
// r + 4 at bit 16 + BITS*r); item pair r of the operand is (code r, code r+4).
//
// Keys, whose scores decide the top-k: each pair becomes exact fp16 integers
// through 1024 + x (OR into 0x6400) minus 1024.  Pairs 0 and 2 are masked at
// bit 0 (x = c); pairs 1 and 3 in place at bit BITS (x = 2^BITS * c, still
// below 1024), so one shift serves two pairs.  The query operand carries
// 2^-BITS on the slots of pairs 1 and 3: every product is then exactly
// c * q, except that a query entry below 2^(BITS-14) in magnitude is rounded
// there (to within 2^(BITS-25)).  The MFMA sums with fp32 rounding only.
template <int BITS>
__device__ inline half8 unpack_keys(uint32_t y) {
  constexpr uint32_t M = ((1u << BITS) - 1) * 0x00010001u;
  // gfx9 VOP3 takes no literal: with the masks in SGPRs and the bias in a
  // VGPR each AND and OR becomes one v_and_or_b32.
  uint32_t m0, m1, bias;
  asm("s_mov_b32 %0, %1" : "=s"(m0) : "i"(M));
  asm("s_mov_b32 %0, %1" : "=s"(m1) : "i"(M << BITS));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(bias));
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t t = y >> (2 * BITS);
  const uint32_t x[4] = {(y & m0) | bias, (y & m1) | bias, (t & m0) | bias, (t & m1) | bias};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x[i]) - k1024);
  return __builtin_bit_cast(half8, r);
}

// MXFP4 keys: E2M1 code c (sign bit 3, magnitude bits e1 e0 m) is the fp16
// pattern ((c & 7) << 9) | ((c & 8) << 12) = its value * 2^-14 exactly (the
// magnitude bits become the exponent's two low bits and the mantissa's top
// bit; index 1, the value 0.5, becomes the subnormal 2^-15).  Pair r is
// (code r, code r + 4) from the nibbles at 4r and 16 + 4r of the key dword.
__device__ inline half8 unpack_keys_mx(uint32_t y) {
  u32x4 r;
  r[0] = ((y << 9) & 0x0E000E00u) | ((y << 12) & 0x80008000u);
  r[1] = ((y << 5) & 0x0E000E00u) | ((y << 8) & 0x80008000u);
  r[2] = ((y << 1) & 0x0E000E00u) | ((y << 4) & 0x80008000u);
  r[3] = ((y >> 3) & 0x0E000E00u) | (y & 0x80008000u);
  return __builtin_bit_cast(half8, r);
}

// INT8 query: the 8 codes of y (as for unpack_keys) as bytes.  4 bits: bytes
// hold channels (0,2,4,6 | 1,3,5,7) -- one AND, one shift and AND; fewer
// bits: (0,1,4,5 | 2,3,6,7).  The query operand takes the same order.
__host__ __device__ constexpr int key_byte_channel(int bits, int i) {
  return (bits == 4) ? ((i & 3) * 2 + (i >> 2)) : ((i & 1) + 4 * ((i >> 1) & 1) + 2 * (i >> 2));
}
template <int BITS>
__device__ inline long unpack_key_bytes(uint32_t y) {
  uint32_t lo, hi;
  if constexpr (BITS == 4) {
    lo = y & 0x0F0F0F0Fu;
    hi = (y >> 4) & 0x0F0F0F0Fu;
  } else {
    constexpr uint32_t M = ((1u << BITS) - 1) * 0x00010001u;
    lo = (y & M) | (((y >> BITS) & M) << 8);
    hi = ((y >> (2 * BITS)) & M) | (((y >> (3 * BITS)) & M) << 8);
  }
  return (long)(((uint64_t)hi << 32) | lo);
}
template <bool Q8>
struct QueryOperand {
  typedef half8 type;
};
template <>
struct QueryOperand<true> {
  typedef long type;
};
// (dependent on KB so that the branch of the other build is not instantiated)
template <int KB>
using QOp = typename QueryOperand<kQ8 && (KB > 0)>::type;
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));

// Key format 2: this lane's B operand of the FP4 scores (column n = query
// head n mod G, K-block kb: 32 E2M1 codes in dwords 0..3) and its E8M0 scale.
struct Fp4Query {
  intx8 b;
  uint32_t sc;
};

// Lane l's value from lane l ^ m of the wave.
__device__ inline int lane_xor(int v, int m, int lane) { return __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, v); }

// Values: the masked bits are used as fp16 bit patterns directly, i.e. the
// subnormals c * 2^(o-24) for a code masked at bit o (patterns below 0x800 are
// linear in their value), which the MFMA multiplies without flushing but sums
// a little less precisely (about 1e-6 of the sum of |products|).  V4: pairs 0
// and 2 at o = 0, pairs 1 and 3 at o = 4 (one shift per two pairs); V2: pair r
// at o = 2r (no shift).  The P operand carries 2^-o on the matching slots and
// the 2^24 is folded into the result.
template <int BITS>
__device__ constexpr int value_slot_exp(int r) { return (BITS == 4) ? 4 * (r & 1) : 2 * r; }
template <int BITS>
__device__ inline half8 unpack_values(uint32_t y) {
  constexpr uint32_t M = (BITS == 4) ? 0x000F000Fu : 0x00030003u;
  u32x4 r;
  if constexpr (BITS == 4) {
    const uint32_t t = y >> 8;
    r[0] = y & M;
    r[1] = y & (M << 4);
    r[2] = t & M;
    r[3] = t & (M << 4);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = y & (M << (2 * i));
  }
  return __builtin_bit_cast(half8, r);
}

__device__ inline float lo_half(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ inline float hi_half(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// a * (fp16 low half of w) as a fused multiply-add with +0: the compiler
// makes it one v_fma_mix (with the fp16 conversion that follows, one
// v_fma_mixlo/mixhi_f16), rounded like the plain product; here a >= 0 and
// the half is a scale >= 0, so the sign of a zero result cannot differ.  A
// plain product would convert the half first and then multiply.  (Not inline
// asm: the compiler does not check hazards inside asm, and this operand comes
// straight from v_exp, whose result needs a wait state before use.)
__device__ inline float mul_lo_half(float a, uint32_t w) { return fmaf(a, lo_half(w), 0.0f); }

__device__ inline uint32_t pack_half2(float lo, float hi) {
  half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));

// The bytes of one 32-token step of one wave, as loaded: every load is a
// whole 1 KB (or 768 B) run of the unit's buffers, lane i taking bytes
// 16i..16i+15 (12i..12i+11 for 3-bit keys), which the layouts make the
// lane's own MFMA operand.
template <int KB, int VB, int G>
struct Step {
  static constexpr int NT = (G == 8) ? 2 : 1;
  uint32_t kc[2][KB];   // key chunk (eighth kb, token 16tt + n): 4 groups x 8 codes
  u32x4 vd[VB / 2];     // value dwords of lane (kb, n), piece-major
  u32x4 meta;           // lane < 32: key meta, else value meta (group, 4 tokens)
};

template <int KB, int VB, int G, bool SIGONLY = false>
__device__ inline void load_step(Step<KB, VB, G>& S, const uint8_t* __restrict__ kbase,
                                 const uint8_t* __restrict__ vbase, const uint32_t* __restrict__ kmeta,
                                 const uint32_t* __restrict__ vmeta, int cap, int t0, int lane, int mshift) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const uint8_t* blk = kbase + (size_t)(t0 / kKBlock + tt) * k_block_bytes(KB) + (size_t)lane * k_chunk_bytes(KB);
    if constexpr (KB == 4) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(blk);
#pragma unroll
      for (int i = 0; i < 4; ++i) S.kc[tt][i] = x[i];
    } else if constexpr (KB == 3) {
      const u32x3 x = *reinterpret_cast<const u32x3*>(blk);
#pragma unroll
      for (int i = 0; i < 3; ++i) S.kc[tt][i] = x[i];
    } else if constexpr (KB == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(blk);
      S.kc[tt][0] = x.x;
      S.kc[tt][1] = x.y;
    } else {
      S.kc[tt][0] = *reinterpret_cast<const uint32_t*>(blk);
    }
  }
  if constexpr (!SIGONLY) {  // (scores only: no values)
    const uint8_t* vt = vbase + (size_t)(t0 / kTile) * v_tile_bytes(VB) + (size_t)lane * 16;
#pragma unroll
    for (int pc = 0; pc < VB / 2; ++pc) S.vd[pc] = *reinterpret_cast<const u32x4*>(vt + 1024 * pc);
  }
  // (key format 2: lanes < 32 read the one plane of key scale words, lanes
  // 8..31 repeating lanes 0..7)
  const size_t plane = (size_t)(((lane & 31) >> 3) >> mshift) * cap;
  const uint32_t* mp = (lane < 32 ? kmeta + (kFP4 ? 0 : plane) : vmeta + plane) + t0 + 4 * (lane & 7);
  if (!SIGONLY || lane < 32) S.meta = *reinterpret_cast<const u32x4*>(mp);
}

// Meta of a step in the wave's LDS slot: 16-byte cells
// [K/V][token tile tt][quarter kb][group g] = the 4 tokens 16tt + 4kb + i.
__device__ inline int meta_cell(int kv, int tt, int kb, int g) { return kv * 32 + tt * 16 + kb * 4 + g; }

// Orders a wave's LDS accesses across its lanes: what some lanes wrote before
// is what other lanes read after (a wave's LDS operations execute in order;
// this keeps the compiler from moving them across each other).
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kSigBatch = 8;  // steps of selection scores staged per wave before a store

// Running softmax state of one wave (see the kernel comment).  ZS distinct
// value-slot scales 2^-o: the sum p * z is kept per scale, x 2^-o.
template <int NT, int ZS>
struct WaveState {
  float m_run;           // running max, log2 units (same in every lane of a head)
  float l_part;          // this lane's share of the denominator
  float z_part[NT][ZS];  // this lane's share of sum p * z for its column (g, h)
  floatx4 acc[8];        // P.V accumulators (x 2^-24: codes enter as fp16 subnormals)
};
template <int VB>
constexpr int kZS = (VB == 4) ? 2 : 4;

// One 32-token step.  MASK: the step straddles the sequence end.  SKIP: the
// tokens whose bit is set in skipw (bit 16tt + 4kb + i for token
// t0 + 16tt + 4kb + i) are left out, as if past the end.  SIGONLY: only the
// selection scores.
template <int KB, int VB, int G, bool MASK, bool SKIP = false, bool SIGONLY = false>
__device__ __forceinline__ void scan_step(const Step<KB, VB, G>& cur, const u32x4 (&km)[2][Step<KB, VB, G>::NT],
                                          const u32x4 (&vm)[Step<KB, VB, G>::NT][2], const uint32_t (&ks)[2],
                                          const Fp4Query& fq, const QOp<KB> (&bq)[kGroups],
                                          const float (&qs)[Step<KB, VB, G>::NT], const float (&qsc)[Step<KB, VB, G>::NT],
                                          WaveState<Step<KB, VB, G>::NT, kZS<VB>>& ws,
                                          floatx4* __restrict__ sig_row, int t0, int len, int n, int kb,
                                          float c_s2, uint32_t skipw = 0) {
  constexpr int NT = Step<KB, VB, G>::NT;
  // -- scores: D[T][tt] rows = tokens 4kb+i of token tile tt, column n --------
  floatx4 d[NT][2];
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) d[T][tt] = (floatx4){0.f, 0.f, 0.f, 0.f};
  intx4 di[NT][2];
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) di[T][tt] = (intx4){0, 0, 0, 0};
#pragma unroll
  for (int tt = 0; tt < 2 && kFP4; ++tt) {  // key format 2: one scaled FP4 MFMA per token tile
    const intx8 a = {(int)cur.kc[tt][0], (int)cur.kc[tt][1], (int)cur.kc[tt][2], (int)cur.kc[tt][3], 0, 0, 0, 0};
    d[0][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, fq.b, d[0][tt], 4, 4, 0, ks[tt], 0, fq.sc);
  }
#pragma unroll
  for (int tt = 0; tt < 2 && !kFP4; ++tt) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      uint32_t y;
      if constexpr (KB == 4) {
        y = cur.kc[tt][g];
      } else if constexpr (KB == 3) {  // 24-bit field g at bit 24g of the 96-bit chunk; codes 4..7 to the high half
        const int d0 = (24 * g) >> 5, d1 = (d0 + 1 < 3) ? d0 + 1 : 2;
        const uint32_t x = __builtin_amdgcn_alignbit(cur.kc[tt][d1], cur.kc[tt][d0], (24 * g) & 31);
        y = (x & 0xFFFFu) | ((x << 4) & 0xFFFF0000u);
      } else if constexpr (KB == 2) {  // 16-bit field g at bit 16g
        const uint32_t x = cur.kc[tt][g >> 1] >> (16 * (g & 1));
        y = (x & 0xFFu) | ((x << 8) & 0x00FF0000u);
      } else {  // 8-bit field g at bit 8g
        const uint32_t x = cur.kc[tt][0] >> (8 * g);
        y = (x & 0xFu) | ((x << 12) & 0x000F0000u);
      }
      const int T = (G == 8) ? (g >> 1) : 0;
      if constexpr (kQ8)
        di[T][tt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(unpack_key_bytes<KB>(y), bq[g], di[T][tt], 0, 0, 0);
      else if constexpr (kMX)
        d[T][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_keys_mx(y), bq[g], d[T][tt], 0, 0, 0);
      else
        d[T][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_keys<KB>(y), bq[g], d[T][tt], 0, 0, 0);
    }
  }
  if constexpr (kQ8) {  // integer sums (|q' . k'| < 2^16: exact) times the query group's scale
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) d[T][tt][i] = (float)di[T][tt][i] * qsc[T];
  }

  // -- per-(token, group) scale and zero, reduce over groups ------------------
  float s2[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float sg4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float part = 0.f;
      if constexpr (kFP4) {
        part = d[0][tt][i];  // the whole logit (both scales applied in the MFMA)
      } else {
#pragma unroll
        for (int T = 0; T < NT; ++T) {
          const uint32_t mw = km[tt][T][i];
          part = fmaf(d[T][tt][i], lo_half(mw), fmaf(hi_half(mw), qs[T], part));
        }
        if constexpr (G == 8) {
          part += dpp<kRowRor8>(part);
        } else {
          part += dpp<kRowRor4>(part);
          part += dpp<kRowRor8>(part);
        }
      }
      if constexpr (MASK) part = ((t0 + 16 * tt + 4 * kb + i) < len) ? part : -INFINITY;
      if constexpr (SKIP) part = ((skipw >> (16 * tt + 4 * kb + i)) & 1u) ? -INFINITY : part;
      // selection score: max over the query heads of the group (the positive
      // factor 1/sqrt(D) commutes with the max and is applied when stored)
      float sg = part;
      sg = fmaxf(sg, dpp<kQuadXor1>(sg));
      sg = fmaxf(sg, dpp<kQuadXor2>(sg));
      if constexpr (G == 8) sg = fmaxf(sg, dpp<kRowRor4>(sg));
      sg4[i] = sg;
      s2[tt][i] = part;  // logit x sqrt(D); x c_s2 gives log2 units
    }
    if (n == 0)
      sig_row[4 * tt + kb] = (floatx4){sg4[0], sg4[1], sg4[2], sg4[3]};
  }
  if constexpr (SIGONLY) return;

  // -- online softmax (log2 units) --------------------------------------------
  // (max(x) * c == max(x * c) for c > 0, rounding included)
  float mloc = fmaxf(fmaxf(fmaxf(s2[0][0], s2[0][1]), fmaxf(s2[0][2], s2[0][3])),
                     fmaxf(fmaxf(s2[1][0], s2[1][1]), fmaxf(s2[1][2], s2[1][3])));
  mloc = max_xor16(mloc);
  mloc = max_xor32(mloc);
  const float m_new = fmaxf(ws.m_run, mloc * c_s2);
  if (__ballot(m_new != ws.m_run)) {  // rare after the first steps
    const float alpha = __builtin_amdgcn_exp2f(ws.m_run - m_new);
    ws.l_part *= alpha;
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int e = 0; e < kZS<VB>; ++e) ws.z_part[T][e] *= alpha;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) ws.acc[nt] *= alpha;
    ws.m_run = m_new;
  }

  // p[tt][r] is the weight x 2^-o of slot r's value scale (see unpack_values)
  // (SKIP can leave a wave with nothing but skipped tokens so far: m_new is
  // then -inf and the reference 0 keeps every weight at exactly 0)
  const float m_ref = (SKIP && m_new == -INFINITY) ? 0.f : m_new;
  float p[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = value_slot_exp<VB>(i);
    const float nm = -m_ref - (float)o;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      p[tt][i] = __builtin_amdgcn_exp2f(fmaf(s2[tt][i], c_s2, nm));
      ws.l_part = (o == 0) ? ws.l_part + p[tt][i] : fmaf(p[tt][i], (float)(1 << o), ws.l_part);
    }
  }

  // -- P.V operand: column (g, h) gets fp16(p * s_g,t); sum p*z on the VALU ---
  half8 bp[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    u32x4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t m0 = vm[T][0][r], m1 = vm[T][1][r];
      if constexpr (MASK) {  // meta past the end may hold anything
        m0 = (t0 + 4 * kb + r) < len ? m0 : 0u;
        m1 = (t0 + 16 + 4 * kb + r) < len ? m1 : 0u;
      }
      float& zr = ws.z_part[T][(VB == 4) ? (r & 1) : r];
      zr = fmaf(p[0][r], hi_half(m0), fmaf(p[1][r], hi_half(m1), zr));
      w[r] = pack_half2(mul_lo_half(p[0][r], m0), mul_lo_half(p[1][r], m1));
    }
    bp[T] = __builtin_bit_cast(half8, w);
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    // column nt: V4 dword nt; V2 dword nt/2 shifted by 8 for odd nt
    const uint32_t y = (VB == 4) ? cur.vd[nt >> 2][nt & 3] : (cur.vd[0][nt >> 1] >> (8 * (nt & 1)));
    const int T = (G == 8) ? (nt >> 2) : 0;
    ws.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(unpack_values<VB>(y), bp[T], ws.acc[nt], 0, 0, 0);
  }
}

// SEL: the launch also selects the top-ksel tokens per unit (the same set
// topk_select finds): each workgroup keeps its split's selection scores in
// LDS, leaves the split's top-min(kk, split length) composites in index order
// in cand, and the unit's last workgroup to finish merges them into idx.
// SKIP: the softmax state leaves out the tokens listed in the first
// min(ksel, len) entries of the unit's row of idx (the workgroup marks those
// of its split in an LDS bitmap first); no selection score is stored.
// SIGONLY: only the selection scores (and SEL's selection): no values are
// read and no split state is written.
// APPEND: first quantise and store the new token of each sequence at
// position len - 1 (what kv_pack_append does for one token): the workgroup
// whose split holds that position does it before its scan reads the cache.
// (The cache pointers carry no __restrict__: this launch writes through them.)
// FUSE: the fused step -- after the scan the same launch selects the unit's
// top-ksel tokens and corrects them into fa.out (fused_tail.h); every
// workgroup of the grid must be resident at once.
// ROWS: the approximate terms of long rows of whole blocks (the rows
// topk_select_blocks writes, ksel entries per unit): workgroup `split` takes
// row entries [split * kRowRec, split * kRowRec + kRowRec), each 32-entry step
// of which is the consecutive tokens t0 .. t0 + nv - 1 of one block (t0 a
// multiple of 32, the entries past the sequence -1), and writes the
// approximate part (max, denominator, value sums) of correction record
// `split` (rcs, records of kCsStride floats, nsplit of them per query head);
// nothing else is written.
template <int KB, int VB, int G, bool SEL, bool SKIP = false, bool SIGONLY = false, bool APPEND = false,
          bool FUSE = false, bool ROWS = false>
__global__ __launch_bounds__(64 * kScanWaves, 8 / kScanWaves) void BKV_SCAN_KERNEL(
    const uint8_t* k_codes, const uint8_t* v_codes, const uint32_t* k_meta, const uint32_t* v_meta,
    const uint16_t* __restrict__ q, float* __restrict__ sigma, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ pacc, SeqArg lens, int Hq, int Hkv, int cap, int nsplit, int chunk,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ counter, int32_t* __restrict__ idx, int ksel, int mshift,
    uint16_t* k_shadow, uint16_t* v_shadow, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, FusedArgs fa, float* __restrict__ rcs) {
  constexpr int NT = Step<KB, VB, G>::NT;
  // (workgroup and lane ids via the builtins: this file is built without IEEE
  // mode, so the device library's id functions would not be inlined)
  const int u = __builtin_amdgcn_workgroup_id_y();
  const int b = u / Hkv;
  const int kvh = u - b * Hkv;
  const int split = __builtin_amdgcn_workgroup_id_x();
  const int len = lens.v[b];
  const int t_begin = split * chunk;
  const int t_end = min(len, t_begin + chunk);
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 15;
  const int kb = lane >> 4;

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  // (key format 2: one plane of scale words per unit)
  const uint32_t* kmeta = k_meta + (size_t)u * (kFP4 ? 1 : meta_planes(mshift)) * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * meta_planes(mshift) * cap;

  // FUSE: the split's histogram of selection scores (fused_tail.h)
  __shared__ uint32_t s_fh[FUSE ? kFBins : 1];
  __shared__ uint32_t s_top;  // FUSE: the highest bin of the split's scores

  // ---- query operands, staged through LDS ------------------------------------
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G][kHeadDim];
  __shared__ float s_qsum[G][kGroups];   // per quarter: sum of q (INT8: s * sum of q')
  __shared__ int8_t s_q8[kQ8 ? G : 1][kHeadDim];  // INT8: the codes q'
  __shared__ float s_qsc[kQ8 ? G : 1][kGroups];   // INT8: the scale s of each quarter's group
  __shared__ __attribute__((aligned(16))) uint32_t s_q4[kFP4 ? G : 1][kGroups][4];  // FP4: codes per quarter
  __shared__ uint32_t s_qe[kFP4 ? G : 1][kGroups];  // FP4: the quarter's E8M0 scale byte
  // Each wave's first step is loaded right after the query row, so that its
  // latency overlaps the prologue below.  The load is unconditional (a
  // clamped, in-range address) so the prologue's wait for the query covers
  // only the query; a wave that has no step, or that appends the new token
  // (its stores must come first), loads again before its first step.
  Step<KB, VB, G> sa, sb, sc;
  int t0 = t_begin + kTile * wv;
  constexpr bool kEarly = !SIGONLY && !ROWS;  // (the scores-only scan keeps two steps in flight: not here)
  bool early = kEarly && t0 < t_end;
  if constexpr (APPEND) {
    const int p = len - 1;
    if (p >= t_begin && p < t_end && wv == (((p - t_begin) >> 5) & (kScanWaves - 1))) early = false;
  }
  {
    const uint4* qg = reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + (size_t)kvh * G) * kHeadDim);
    const uint4 qv = qg[tid % (G * kHeadDim / 8)];
    if constexpr (kEarly)
      load_step<KB, VB, G, SIGONLY>(sa, kbase, vbase, kmeta, vmeta, cap, min(t0, cap - kTile), lane, mshift);
    if (tid < G * kHeadDim / 8) reinterpret_cast<uint4*>(&s_q[0][0])[tid] = qv;
    if constexpr (FUSE) {  // the split's score histogram starts empty
      for (int i = tid; i < kFBins; i += 64 * kScanWaves) s_fh[i] = 0u;
      if (tid == 0) s_top = 0u;
    }
    __syncthreads();
    if constexpr (kQ8) {
      // one entry per thread, whole waves: a wave holds 64 channels of one head,
      // a group is 32 << mshift of its lanes
      for (int e = tid; e < G * kHeadDim; e += 64 * kScanWaves) {
        const int hh = e / kHeadDim, c = e % kHeadDim;
        const float x = (float)__builtin_bit_cast(_Float16, s_q[hh][c]);
        float a = fabsf(x);
        for (int m = 1; m < (kGroup << mshift); m <<= 1) a = fmaxf(a, __int_as_float(lane_xor(__float_as_int(a), m, lane)));
        const float sc = query_scale_i8(a);
        const int code = query_code_i8(x, sc);
        s_q8[hh][c] = (int8_t)code;
        int sum = code;
        for (int m = 1; m < kGroup; m <<= 1) sum += lane_xor(sum, m, lane);
        if ((c & (kGroup - 1)) == 0) {
          s_qsum[hh][c / kGroup] = sc * (float)sum;
          s_qsc[hh][c / kGroup] = sc;
        }
      }
    } else if constexpr (kFP4) {
      // a quad of threads per (head, quarter), 8 channels each: the same
      // rule as the keys' (whole waves: G * 16 is 64 or 128)
      if (tid < G * 16) {
        const int hh = tid >> 4, grp = (tid >> 2) & 3, sub = tid & 3;
        float x[8];
        halves8(*reinterpret_cast<const uint4*>(&s_q[hh][grp * kGroup + 8 * sub]), x);
        uint32_t code[8];
        const uint32_t e8 = quantise_lane_e8(x, code);
        uint32_t f = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) f |= code[j] << (4 * j);
        s_q4[hh][grp][sub] = f;
        if (sub == 0) s_qe[hh][grp] = e8;
      }
    } else if (tid < G * kGroups) {
      const int hh = tid / kGroups, g = tid % kGroups;
      float s = 0.f;
      for (int c = 0; c < kGroup; ++c) s += (float)__builtin_bit_cast(_Float16, s_q[hh][g * kGroup + c]);
      s_qsum[hh][g] = s;
    }
    __syncthreads();
  }
  if constexpr (APPEND) {
    const int p = len - 1;  // the new token
    // The wave whose steps hold it quantises and stores it before its first
    // load and waits for its own stores (the step with the token is its
    // last, and no other wave reads that step); the other waves start
    // scanning at once.
    if (p >= t_begin && p < t_end && wv == (((p - t_begin) >> 5) & (kScanWaves - 1))) {
      __shared__ uint8_t s_newv[kHeadDim];  // its value codes
      if (lane < 32) {  // 16 lanes for K, 16 for V, four per quarter
        const int sub = lane & 3, grp = (lane >> 2) & 3, kv = (lane >> 4) & 1;
        const int c0 = grp * kGroup + sub * 8;
        const uint4 w4 = *reinterpret_cast<const uint4*>((kv ? v_new : k_new) + (size_t)u * kHeadDim + c0);
        float x[8];
        halves8(w4, x);
        uint32_t code[8];
        const uint32_t mw = (kMX && kv == 0)    ? quantise_lane_mx(x, code)
                            : (kFP4 && kv == 0) ? quantise_lane_e8(x, code)
                                                : quantise_lane(x, sub, grp, mshift, (float)((1 << (kv ? VB : KB)) - 1), code);
        if (kFP4 && kv == 0) {
          if (sub == 0)
            reinterpret_cast<uint8_t*>(const_cast<uint32_t*>(k_meta))[((size_t)u * cap + p) * kGroups + grp] = (uint8_t)mw;
        } else if (sub == 0 && (grp & ((1 << mshift) - 1)) == 0) {
          const_cast<uint32_t*>(kv ? v_meta : k_meta)[((size_t)u * meta_planes(mshift) + (grp >> mshift)) * cap + p] =
              mw;
        }
        *reinterpret_cast<uint4*>((kv ? v_shadow : k_shadow) + ((size_t)u * cap + p) * kHeadDim + c0) = w4;
        if (kv == 0) {
          if constexpr (kFP4)
            store_key_codes_e8(const_cast<uint8_t*>(k_codes) + (size_t)u * k_unit_bytes(KB, cap), p, sub, grp, code);
          else
            store_key_codes<KB>(const_cast<uint8_t*>(k_codes) + (size_t)u * k_unit_bytes(KB, cap), p, sub, grp, code);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) s_newv[c0 + j] = (uint8_t)code[j];
        }
      }
      wave_lds_order();
      // its slot in the value tile: token r is in quarter qq = (r mod 16)/4 at
      // slot j; lanes 16qq..16qq+15 of the tile hold it, each in 2*VB dwords
      // of 4/VB columns (32*VB dwords, two per lane of this wave for V4)
      constexpr int kCpd = 4 / VB;
      const int r = p % kTile, qq = (r & 15) >> 2, j = 4 * (r >> 4) + (r & 3);
      uint32_t* vt = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(v_codes) + (size_t)u * v_unit_bytes(VB, cap) +
                                                 (size_t)(p / kTile) * v_tile_bytes(VB));
      for (int e = lane; e < 32 * VB; e += 64) {
        const int l = 16 * qq + (e & 15), d = e >> 4;
        const int dw = 256 * (d >> 2) + 4 * l + (d & 3);
        uint32_t word = vt[dw];
#pragma unroll
        for (int sb = 0; sb < kCpd; ++sb) {
          const int c = 16 * (d * kCpd + sb) + (l & 15);
          const int bit = 16 * (j >> 2) + 4 * VB * sb + VB * (j & 3);
          const uint32_t m = ((1u << VB) - 1) << bit;
          word = (word & ~m) | ((uint32_t)s_newv[c] << bit);
        }
        vt[dw] = word;
      }
      __builtin_amdgcn_s_waitcnt(0);  // (its stores are done before this wave loads the step)
    }
  }
  // SKIP: bit t - t_begin marks a listed token of the split
  __shared__ uint32_t s_skip[SKIP ? kSelStage / 32 : 1];
  if constexpr (SKIP) {
    for (int i = tid; i < kSelStage / 32; i += 64 * kScanWaves) s_skip[i] = 0u;
    __syncthreads();
    const int kk = min(ksel, len);
    const int32_t* row = idx + (size_t)u * ksel;
    for (int j = tid; j < kk; j += 64 * kScanWaves) {
      const int t = row[j];
      if (t >= t_begin && t < t_end) atomicOr(&s_skip[(t - t_begin) >> 5], 1u << ((t - t_begin) & 31));
    }
    __syncthreads();
  }
  // column (g', h) of N-tile T: g' = n/4 (G = 4) or 2T + n/8 (G = 8)
  const int h = (G == 8) ? (n & 7) : (n & 3);
  QOp<KB> bq[kGroups];
  float qs[NT], qsc[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int gq = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
    qs[T] = s_qsum[h][gq];
    if constexpr (kQ8)
      qsc[T] = s_qsc[h][gq];
    else
      qsc[T] = 1.0f;
  }
  Fp4Query fq;  // key format 2: column n = head h, K-block kb
  fq.b = (intx8){0, 0, 0, 0, 0, 0, 0, 0};
  fq.sc = 127u;
  if constexpr (kFP4) {
    const uint4 w = *reinterpret_cast<const uint4*>(&s_q4[h][kb][0]);
    fq.b = (intx8){(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    fq.sc = s_qe[h][kb];
  }
#pragma unroll
  for (int g = 0; g < kGroups && !kFP4; ++g) {
    const int gq = (G == 8) ? (2 * (g >> 1) + (n >> 3)) : (n >> 2);
    if constexpr (kQ8) {  // the codes of channels 32g + 8kb + key_byte_channel(i), in column (g, h) only
      uint64_t v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v |= (uint64_t)(uint8_t)s_q8[h][g * kGroup + 8 * kb + key_byte_channel(KB, i)] << (8 * i);
      bq[g] = (gq == g) ? (long)v : 0l;
      continue;
    } else {
    half8 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // slots of pairs 1 and 3 carry 2^-KB (see unpack_keys)
      const float sc = ((r & 1) && !kMX) ? 1.0f / (float)(1 << KB) : 1.0f;
      const float q0 = (float)__builtin_bit_cast(_Float16, s_q[h][g * kGroup + 8 * kb + r]);
      const float q1 = (float)__builtin_bit_cast(_Float16, s_q[h][g * kGroup + 8 * kb + 4 + r]);
      v[2 * r] = (gq == g) ? (_Float16)(q0 * sc) : (_Float16)0.0f;
      v[2 * r + 1] = (gq == g) ? (_Float16)(q1 * sc) : (_Float16)0.0f;
    }
    bq[g] = v;
    }
  }

  // (MXFP4 keys: the MFMA saw values * 2^-14)
  const float sm = (1.0f / sqrtf((float)kHeadDim)) * (kMX ? 16384.0f : 1.0f);
  const float c_sig = sm;
  const float c_s2 = sm * kLog2e;
  float* sig = sigma + (size_t)u * cap;

  WaveState<NT, kZS<VB>> ws;
  ws.m_run = -INFINITY;
  ws.l_part = 0.f;
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int e = 0; e < kZS<VB>; ++e) ws.z_part[T][e] = 0.f;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) ws.acc[nt] = (floatx4){0.f, 0.f, 0.f, 0.f};

  // per-wave LDS slot for the step's meta (each wave only touches its own)
  __shared__ u32x4 s_meta[kScanWaves][64];
  u32x4* slot = s_meta[wv];
  const int wcell = meta_cell(lane >> 5, (lane & 7) >> 2, lane & 3, (lane & 31) >> 3);

  // Selection scores go through a per-wave LDS buffer of kSigBatch steps and
  // leave as one coalesced 16-byte-per-lane store (no stores in the steps).
  __shared__ floatx4 s_sig[kScanWaves][kSigBatch][8];
  // SEL, FUSE: the split's selection scores, as stored ([t - t_begin])
  __shared__ __attribute__((aligned(16))) float s_split[(SEL || FUSE) ? kSelStage : 1];
  uint32_t fmaxb = 0;  // FUSE: this lane's highest bin so far
  int sig_count = 0;   // steps staged
  int sig_first = 0;   // t0 of the first staged step
  auto flush_sig = [&]() {
    wave_lds_order();
    const int i = lane >> 3;
    if (i < sig_count) {
      const int t = sig_first + kScanWaves * kTile * i + 4 * (lane & 7);
      const floatx4 v = s_sig[wv][i][lane & 7] * c_sig;
      if constexpr (!SKIP) *reinterpret_cast<floatx4*>(sig + t) = v;
      if constexpr (SEL || FUSE) *reinterpret_cast<floatx4*>(&s_split[t - t_begin]) = v;
      if constexpr (FUSE) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (t + x < t_end) {
            const uint32_t bn = fbin(v[x]);
            atomicAdd(&s_fh[bn], 1u);
            fmaxb = max(fmaxb, bn);
          }
        }
      }
    }
    wave_lds_order();
    sig_count = 0;
  };

  // Meta of the step -> this lane's cells: lane (n, kb) needs its column's
  // group for tokens 16tt + 4kb + i.
  // Key format 2: lane (n, kb) takes the scale word of token 16tt + n (cell
  // (K, tt, n/4, 0), entry n mod 4) and its byte kb (the MFMA reads the low
  // byte of its scale operand).
  auto meta_cells = [&](const u32x4& meta, u32x4 (&km)[2][NT], u32x4 (&vm)[NT][2], uint32_t (&ks)[2]) {
    wave_lds_order();  // the previous step's reads of the slot come first
    slot[wcell] = meta;
    wave_lds_order();
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const int gq = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if constexpr (!kFP4) km[tt][T] = slot[meta_cell(0, tt, kb, gq)];
        vm[T][tt] = slot[meta_cell(1, tt, kb, gq)];
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      ks[tt] = kFP4 ? reinterpret_cast<const uint32_t*>(slot)[4 * meta_cell(0, tt, n >> 2, 0) + (n & 3)] >> (8 * kb)
                    : 0u;
  };

  // One whole step: prefetch the wave's step kAhead steps on into `nxt`
  // (unconditionally -- past the end it re-reads this step's bytes -- so that
  // the compiler's wait for this step's data counts those loads), then score
  // and accumulate `cur`.  The loop is unrolled kAhead + 1 times so the
  // register sets rotate without copies (a copy of registers with loads in
  // flight would wait for them).  Scores only (keys only, small steps): two
  // steps in flight; otherwise one (two measured slower there).
  constexpr int kAhead = SIGONLY ? 2 : 1;
  auto full_step = [&](Step<KB, VB, G>& cur, Step<KB, VB, G>& nxt, int t0) {
    const int tn = (t0 + kAhead * kScanWaves * kTile) < t_end ? t0 + kAhead * kScanWaves * kTile : t0;
    load_step<KB, VB, G, SIGONLY>(nxt, kbase, vbase, kmeta, vmeta, cap, tn, lane, mshift);
    u32x4 km[2][NT], vm[NT][2];
    uint32_t ks[2];
    meta_cells(cur.meta, km, vm, ks);
    if (sig_count == 0) sig_first = t0;
    scan_step<KB, VB, G, false, SKIP, SIGONLY>(cur, km, vm, ks, fq, bq, qs, qsc, ws, s_sig[wv][sig_count], t0, len, n, kb, c_s2,
                                      SKIP ? s_skip[(t0 - t_begin) >> 5] : 0u);
    if (++sig_count == kSigBatch) flush_sig();
  };
  // The step that straddles the end of the split (at most one per wave).
  auto last_step = [&](Step<KB, VB, G>& cur, int t0) {
    u32x4 km[2][NT], vm[NT][2];
    uint32_t ks[2];
    meta_cells(cur.meta, km, vm, ks);
    if (sig_count == 0) sig_first = t0;
    scan_step<KB, VB, G, true, SKIP, SIGONLY>(cur, km, vm, ks, fq, bq, qs, qsc, ws, s_sig[wv][sig_count], t0, t_end, n, kb, c_s2,
                                     SKIP ? s_skip[(t0 - t_begin) >> 5] : 0u);
    ++sig_count;
  };
  if constexpr (ROWS) {
    // the wave's two steps of the record (kRowRec = 16 steps of 32 entries):
    // first token and count of each, then both loads in flight at once (a
    // step with no token loads token 0's step and is not scanned)
    static_assert(kRowRec == 2 * kScanWaves * kTile, "two steps per wave");
    const int32_t* rowp = idx + (size_t)u * ksel;
    const int kk = min(ksel, len);
    const int r_begin = split * kRowRec, r_end = min(kk, r_begin + kRowRec);
    if (r_begin >= kk) return;  // (the whole workgroup: the combine reads only the records below kk)
    int rt0[2], rnv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e0 = r_begin + kTile * (wv + kScanWaves * i);
      const int e = e0 + (lane & 31);
      const int v = (e < r_end) ? rowp[e] : -1;
      const uint64_t okm = __ballot(v >= 0 && v < len) & 0xFFFFFFFFull;
      rnv[i] = __builtin_amdgcn_readfirstlane(__popcll(okm));
      rt0[i] = __builtin_amdgcn_readfirstlane((v >= 0 && v < len) ? v : 0) & ~(kTile - 1);
    }
    load_step<KB, VB, G, false>(sa, kbase, vbase, kmeta, vmeta, cap, rt0[0], lane, mshift);
    load_step<KB, VB, G, false>(sb, kbase, vbase, kmeta, vmeta, cap, rt0[1], lane, mshift);
    auto rows_step = [&](const Step<KB, VB, G>& cur, int ts, int nv) {
      u32x4 km[2][NT], vm[NT][2];
      uint32_t ks[2];
      meta_cells(cur.meta, km, vm, ks);
      if (nv == kTile)
        scan_step<KB, VB, G, false>(cur, km, vm, ks, fq, bq, qs, qsc, ws, s_sig[wv][0], ts, ts + nv, n, kb, c_s2);
      else if (nv > 0)
        scan_step<KB, VB, G, true>(cur, km, vm, ks, fq, bq, qs, qsc, ws, s_sig[wv][0], ts, ts + nv, n, kb, c_s2);
    };
    rows_step(sa, rt0[0], rnv[0]);
    rows_step(sb, rt0[1], rnv[1]);
  } else if constexpr (kAhead == 1) {
    if (t0 < t_end && !early) load_step<KB, VB, G, SIGONLY>(sa, kbase, vbase, kmeta, vmeta, cap, t0, lane, mshift);
    for (;;) {
      if (t0 + kTile > t_end) {
        if (t0 < t_end) last_step(sa, t0);
        break;
      }
      full_step(sa, sb, t0);
      t0 += kScanWaves * kTile;
      if (t0 + kTile > t_end) {
        if (t0 < t_end) last_step(sb, t0);
        break;
      }
      full_step(sb, sa, t0);
      t0 += kScanWaves * kTile;
    }
  } else {
  if (t0 < t_end) {
    load_step<KB, VB, G, SIGONLY>(sa, kbase, vbase, kmeta, vmeta, cap, t0, lane, mshift);
    const int t1 = (t0 + kScanWaves * kTile) < t_end ? t0 + kScanWaves * kTile : t0;
    load_step<KB, VB, G, SIGONLY>(sb, kbase, vbase, kmeta, vmeta, cap, t1, lane, mshift);
  }
  for (;;) {
    if (t0 + kTile > t_end) {
      if (t0 < t_end) last_step(sa, t0);
      break;
    }
    full_step(sa, sc, t0);
    t0 += kScanWaves * kTile;
    if (t0 + kTile > t_end) {
      if (t0 < t_end) last_step(sb, t0);
      break;
    }
    full_step(sb, sa, t0);
    t0 += kScanWaves * kTile;
    if (t0 + kTile > t_end) {
      if (t0 < t_end) last_step(sc, t0);
      break;
    }
    full_step(sc, sb, t0);
    t0 += kScanWaves * kTile;
  }
  }
  if (sig_count > 0) flush_sig();

  // ---- combine the waves of the workgroup -----------------------------------
  if constexpr (SIGONLY) {
    __syncthreads();  // (orders every flush before the selection below)
  } else {
  ws.l_part += __shfl_xor(ws.l_part, 16);
  ws.l_part += __shfl_xor(ws.l_part, 32);
  float z_tot[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < kZS<VB>; ++e) z = fmaf(ws.z_part[T][e], (float)(1 << value_slot_exp<VB>(e)), z);
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    z_tot[T] = z;
  }
  __shared__ float s_m[kScanWaves][G];
  __shared__ float s_l[kScanWaves][G];
  __shared__ float s_acc[kScanWaves][G][kHeadDim];
  if (kb == 0 && n < G) {
    s_m[wv][h] = ws.m_run;
    s_l[wv][h] = ws.l_part;
  }
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int g = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nt = 2 * g + j;
      // nt is lane dependent; select the accumulator without dynamic indexing
      floatx4 a = ws.acc[0];
#pragma unroll
      for (int x = 1; x < 8; ++x)
        if (x == nt) a = ws.acc[x];
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[wv][h][16 * nt + 4 * kb + i] = fmaf(a[i], 0x1p24f, z_tot[T]);
    }
  }
  __syncthreads();

  constexpr int NR = G * kHeadDim / (64 * kScanWaves);  // (head, channel) pairs per thread
  float rm[NR], rl[NR], ra[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = tid + 64 * kScanWaves * r;
    const int hh = e / kHeadDim;
    const int c = e - hh * kHeadDim;
    float M = s_m[0][hh];
#pragma unroll
    for (int x = 1; x < kScanWaves; ++x) M = fmaxf(M, s_m[x][hh]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int x = 0; x < kScanWaves; ++x) {
        const float f = __builtin_amdgcn_exp2f(s_m[x][hh] - M);
        a += f * s_acc[x][hh][c];
        l += f * s_l[x][hh];
      }
    }
    if constexpr (FUSE) {
      rm[r] = M;
      rl[r] = l;
      ra[r] = a;
    } else if constexpr (ROWS) {  // the record's approximate part
      float* rr = rcs + (((size_t)b * Hq + (size_t)kvh * G + hh) * nsplit + split) * kCsStride;
      rr[4 + kHeadDim + c] = a;
      if (c == 0) {
        rr[2] = M;
        rr[3] = l;
      }
    } else {
      const size_t rec = ((size_t)b * Hq + (size_t)kvh * G + hh) * nsplit + split;
      pacc[rec * kHeadDim + c] = a;
      if (c == 0) {
        pm[rec] = M;
        pl[rec] = l;
      }
    }
  }
  if constexpr (FUSE) {
    {  // the split's top bin (bins are below 2^13: exact as floats)
      const float wm = wave_minmax<true>((float)fmaxb);
      if (lane == 0) atomicMax(&s_top, (uint32_t)wm);
      __syncthreads();
    }
    FusedCtx<G> x;
    x.top_bin = s_top;
    x.tid = tid;
    x.u = u;
    x.b = b;
    x.kvh = kvh;
    x.split = split;
    x.len = len;
    x.t_begin = t_begin;
    x.t_end = t_end;
    x.nsplit = nsplit;
    x.chunk = chunk;
    x.ksel = ksel;
    x.cap = cap;
    x.mshift = mshift;
    x.Hq = Hq;
    x.kbase = kbase;
    x.vbase = vbase;
    x.kmeta = kmeta;
    x.vmeta = vmeta;
    x.ksh = k_shadow + (size_t)u * cap * kHeadDim;
    x.vsh = v_shadow + (size_t)u * cap * kHeadDim;
    x.pm = pm;
    x.pl = pl;
    x.pacc = pacc;
    x.idx = idx;
    x.fa = fa;
    x.s_q = s_q;
    x.s_split = s_split;
    x.s_fh = s_fh;
    x.s_acc = &s_acc[0][0][0];
    x.s_lg = reinterpret_cast<float*>(&s_meta[0][0]);
    x.s_w = reinterpret_cast<float*>(&s_sig[0][0][0]);
    fused_tail<KB, VB, G, kFP4 ? 2 : (kMX ? 1 : 0)>(x, rm, rl, ra);
    return;
  }
  }  // !SIGONLY

  if constexpr (SEL) {
    // ---- the split's top-min(kk, split length), then the unit's merge -----------
    // (the barrier above ordered every flush before these reads)
    constexpr int NT = 64 * kScanWaves;
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ int s_wsum[kScanWaves];
    __shared__ int s_res[4];
    __shared__ int s_last;
    __shared__ float s_mm[2 * kScanWaves];
    __shared__ uint64_t s_small[65];
    const int kk = min(ksel, len);
    const int len_s = max(0, t_end - t_begin);
    uint64_t* __restrict__ ucand = cand + (size_t)u * nsplit * ksel;
    if (0 < kk && kk < len && len_s > 0) {
      const int cnt = min(kk, len_s);
      // thread tid holds entries j*NT + tid in registers (0: past the range)
      constexpr int PER = kSelStage / NT;
      uint64_t c[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = j * NT + tid;
        c[j] = (i < len_s) ? composite(s_split[i], t_begin + i) : 0ull;
      }
      auto get = [&](int i) { return composite(s_split[i], t_begin + i); };
      auto fill = [] {};  // the scores are in LDS already
      const uint64_t T = (cnt == len_s) ? 0
                                        : hist_select<NT>(c, len_s, cnt, get, fill, s_hist, s_wsum, s_res, s_mm,
                                                          s_small);
      // the entries >= T in index order (entry j*NT + 64w + lane is (j, w, lane))
      bool sel[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) sel[j] = c[j] && c[j] >= T;
      int at[PER];
      ordered_positions<PER, kScanWaves>(sel, at, s_wsum, reinterpret_cast<int*>(s_hist));
      uint64_t* __restrict__ dst = ucand + (size_t)split * ksel;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (sel[j]) st_dev64(&dst[at[j]], c[j]);
      for (int j = cnt + tid; j < ksel; j += NT) st_dev64(&dst[j], 0ull);  // the split's unused slots
    }
    if (!arrive_is_last(&counter[u], (uint32_t)nsplit, &s_last)) return;
    merge_unit<NT, true, kSelSlots>(ucand, idx, u, len, 0, ksel, 0, chunk, reinterpret_cast<uint64_t*>(s_split),
                                    s_hist, s_wsum, s_res, s_mm, s_small);
    if (tid == 0) counter[u] = 0u;  // ready for the next call on this workspace
  }
}

template <int KB, int VB, int G>
hipError_t launch_t(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                    float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel, bool skip, bool sigonly,
                    const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  dim3 grid(w.nsplit, L.batch * L.n_kv_heads);
  const int mshift = L.group == 64 ? 1 : 0;
  const uint8_t* kc = static_cast<const uint8_t*>(c.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(c.v_codes);
  (void)hipGetLastError();  // report only this launch's status
  if (k_new && ksel > 0)
    BKV_SCAN_KERNEL<KB, VB, G, true, false, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, w.tkc, w.tkctr, idx, ksel, mshift, c.k_shadow, c.v_shadow, k_new, v_new, FusedArgs{}, nullptr);
  else if (k_new)
    BKV_SCAN_KERNEL<KB, VB, G, false, false, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, nullptr, nullptr, nullptr, 0, mshift, c.k_shadow, c.v_shadow, k_new, v_new, FusedArgs{}, nullptr);
  else if (sigonly && ksel > 0)
    BKV_SCAN_KERNEL<KB, VB, G, true, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, nullptr, nullptr, nullptr, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, w.tkc, w.tkctr, idx, ksel, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, nullptr);
  else if (sigonly)
    BKV_SCAN_KERNEL<KB, VB, G, false, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, nullptr, nullptr, nullptr, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, nullptr, nullptr, nullptr, 0, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, nullptr);
  else if (skip)
    BKV_SCAN_KERNEL<KB, VB, G, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, nullptr, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, nullptr, nullptr, idx, ksel, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, nullptr);
  else if (ksel > 0)
    BKV_SCAN_KERNEL<KB, VB, G, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, w.tkc, w.tkctr, idx, ksel, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, nullptr);
  else
    BKV_SCAN_KERNEL<KB, VB, G, false><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, nullptr, nullptr, nullptr, 0, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, nullptr);
  return hipGetLastError();
}


// Resident workgroups of a launch of fn (512 threads) on the current device,
// or 0 if unknown.
static int resident_workgroups(const void* fn, int& cache) {
  int per = cache;
  if (per == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, 64 * kScanWaves, 0) != hipSuccess) return 0;
    cache = per;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per * cus;
}

// Whether the fused grid (nsplit x units workgroups) is resident on the
// current device at once, as the unit barriers need.
template <int KB, int VB, int G>
bool fused_fits_t(const bkv_layout& L, const Workspace& w, bool append) {
  static int occ_append = 0, occ_plain = 0;  // (per kernel; the same on every device of this build)
  const void* fn = append ? reinterpret_cast<const void*>(&BKV_SCAN_KERNEL<KB, VB, G, false, false, false, true, true>)
                          : reinterpret_cast<const void*>(&BKV_SCAN_KERNEL<KB, VB, G, false, false, false, false, true>);
  return (long long)resident_workgroups(fn, append ? occ_append : occ_plain) >=
         (long long)w.nsplit * L.batch * L.n_kv_heads;
}

template <int KB, int VB, int G>
hipError_t launch_fused_t(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                          float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel, const uint16_t* k_new,
                          const uint16_t* v_new, float* out, hipStream_t s) {
  const dim3 grid(w.nsplit, L.batch * L.n_kv_heads);
  const int mshift = L.group == 64 ? 1 : 0;
  const uint8_t* kc = static_cast<const uint8_t*>(c.k_codes);
  const uint8_t* vc = static_cast<const uint8_t*>(c.v_codes);
  FusedArgs fa = w.fused;
  fa.out = out;
  // the unit barriers need every workgroup resident at once
  if (!fused_fits_t<KB, VB, G>(L, w, k_new != nullptr)) return hipErrorNotSupported;
  (void)hipGetLastError();  // report only this launch's status
  if (k_new)
    BKV_SCAN_KERNEL<KB, VB, G, false, false, false, true, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, w.tkc, nullptr, idx, ksel, mshift, c.k_shadow, c.v_shadow, k_new, v_new, fa, nullptr);
  else
    BKV_SCAN_KERNEL<KB, VB, G, false, false, false, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
        kc, vc, c.k_meta, c.v_meta, q, sigma, w.part.m, w.part.l, w.part.acc, len, L.n_q_heads, L.n_kv_heads,
        L.capacity, w.nsplit, chunk, w.tkc, nullptr, idx, ksel, mshift, c.k_shadow, c.v_shadow, nullptr, nullptr, fa, nullptr);
  return hipGetLastError();
}

// ROWS: the approximate parts of the nrec correction records of long rows.
template <int KB, int VB, int G>
hipError_t launch_rows_t(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                         const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s) {
  const dim3 grid(nrec, L.batch * L.n_kv_heads);
  const int mshift = L.group == 64 ? 1 : 0;
  (void)hipGetLastError();  // report only this launch's status
  BKV_SCAN_KERNEL<KB, VB, G, false, false, false, false, false, true><<<grid, 64 * kScanWaves, 0, s>>>(
      static_cast<const uint8_t*>(c.k_codes), static_cast<const uint8_t*>(c.v_codes), c.k_meta, c.v_meta, q, nullptr,
      nullptr, nullptr, nullptr, len, L.n_q_heads, L.n_kv_heads, L.capacity, w.nchunk, kRowRec, nullptr, nullptr,
      const_cast<int32_t*>(idx), row, mshift, nullptr, nullptr, nullptr, nullptr, FusedArgs{}, w.cs);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_rows_g(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                         const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s) {
  if (L.n_q_heads / L.n_kv_heads == 4) return launch_rows_t<KB, VB, 4>(L, c, q, len, w, idx, row, nrec, s);
  return launch_rows_t<KB, VB, 8>(L, c, q, len, w, idx, row, nrec, s);
}

template <int KB, int VB>
hipError_t launch_g(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                    float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel, bool skip, bool sigonly,
                    const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  const int G = L.n_q_heads / L.n_kv_heads;
  if (G == 4) return launch_t<KB, VB, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
  return launch_t<KB, VB, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
}

}  // namespace

#if BKV_KEY_MXFP4 || BKV_KEY_FP4
// The fused step of the MXFP4 key formats (4-bit keys), this build's.
#if BKV_KEY_FP4
#define BKV_FUSED_FITS decode_fused_fits_fp4
#define BKV_FUSED_LAUNCH launch_decode_fused_fp4
#else
#define BKV_FUSED_FITS decode_fused_fits_mx
#define BKV_FUSED_LAUNCH launch_decode_fused_mx
#endif
bool BKV_FUSED_FITS(const bkv_layout& L, const Workspace& w, bool append) {
  const bool g4 = L.n_q_heads / L.n_kv_heads == 4;
  if (L.v_bits == 4) return g4 ? fused_fits_t<4, 4, 4>(L, w, append) : fused_fits_t<4, 4, 8>(L, w, append);
  return g4 ? fused_fits_t<4, 2, 4>(L, w, append) : fused_fits_t<4, 2, 8>(L, w, append);
}
hipError_t BKV_FUSED_LAUNCH(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                            float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel,
                            const uint16_t* k_new, const uint16_t* v_new, float* out, hipStream_t s) {
  const bool g4 = L.n_q_heads / L.n_kv_heads == 4;
  if (L.v_bits == 4)
    return g4 ? launch_fused_t<4, 4, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
              : launch_fused_t<4, 4, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
  return g4 ? launch_fused_t<4, 2, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
            : launch_fused_t<4, 2, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
}
#endif

#if !BKV_QUERY_INT8 && !BKV_KEY_MXFP4 && !BKV_KEY_FP4
// (dispatch to the build of the layout's key format)
bool decode_fused_fits(const bkv_layout& L, const Workspace& w, bool append) {
  if (L.query_bits != 0 || L.k_bits < 3) return false;
  if (L.key_format == 1) return L.k_bits == 4 && decode_fused_fits_mx(L, w, append);
  if (L.key_format == 2) return L.k_bits == 4 && decode_fused_fits_fp4(L, w, append);
  const bool g4 = L.n_q_heads / L.n_kv_heads == 4;
  const bool v4 = L.v_bits == 4;
  if (L.k_bits == 4) {
    if (v4) return g4 ? fused_fits_t<4, 4, 4>(L, w, append) : fused_fits_t<4, 4, 8>(L, w, append);
    return g4 ? fused_fits_t<4, 2, 4>(L, w, append) : fused_fits_t<4, 2, 8>(L, w, append);
  }
  if (v4) return g4 ? fused_fits_t<3, 4, 4>(L, w, append) : fused_fits_t<3, 4, 8>(L, w, append);
  return g4 ? fused_fits_t<3, 2, 4>(L, w, append) : fused_fits_t<3, 2, 8>(L, w, append);
}

hipError_t launch_decode_fused(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                               float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel,
                               const uint16_t* k_new, const uint16_t* v_new, float* out, hipStream_t s) {
  if (L.query_bits != 0 || L.k_bits < 3) return hipErrorNotSupported;
  if (L.key_format == 1 || L.key_format == 2) {
    if (L.k_bits != 4) return hipErrorNotSupported;
    return L.key_format == 1 ? launch_decode_fused_mx(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
                             : launch_decode_fused_fp4(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
  }
  const bool g4 = L.n_q_heads / L.n_kv_heads == 4;
  const bool v4 = L.v_bits == 4;
  if (L.k_bits == 4) {
    if (v4) return g4 ? launch_fused_t<4, 4, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
                      : launch_fused_t<4, 4, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
    return g4 ? launch_fused_t<4, 2, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
              : launch_fused_t<4, 2, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
  }
  if (v4) return g4 ? launch_fused_t<3, 4, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
                    : launch_fused_t<3, 4, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
  return g4 ? launch_fused_t<3, 2, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s)
            : launch_fused_t<3, 2, 8>(L, c, q, len, sigma, w, chunk, idx, ksel, k_new, v_new, out, s);
}
#endif

hipError_t BKV_ROWS_LAUNCH(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                           const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s) {
#if !BKV_QUERY_INT8 && !BKV_KEY_MXFP4 && !BKV_KEY_FP4
  if (L.query_bits == 8) return launch_rows_approx_q8(L, c, q, len, w, idx, row, nrec, s);
  if (L.key_format == 1) return launch_rows_approx_mx(L, c, q, len, w, idx, row, nrec, s);
  if (L.key_format == 2) return launch_rows_approx_fp4(L, c, q, len, w, idx, row, nrec, s);
#endif
#if BKV_KEY_MXFP4 || BKV_KEY_FP4  // (4-bit keys only)
  return L.v_bits == 4 ? launch_rows_g<4, 4>(L, c, q, len, w, idx, row, nrec, s)
                       : launch_rows_g<4, 2>(L, c, q, len, w, idx, row, nrec, s);
#else
  const bool v4 = L.v_bits == 4;
  switch (L.k_bits) {
    case 4: return v4 ? launch_rows_g<4, 4>(L, c, q, len, w, idx, row, nrec, s) : launch_rows_g<4, 2>(L, c, q, len, w, idx, row, nrec, s);
    case 3: return v4 ? launch_rows_g<3, 4>(L, c, q, len, w, idx, row, nrec, s) : launch_rows_g<3, 2>(L, c, q, len, w, idx, row, nrec, s);
    case 2: return v4 ? launch_rows_g<2, 4>(L, c, q, len, w, idx, row, nrec, s) : launch_rows_g<2, 2>(L, c, q, len, w, idx, row, nrec, s);
    default: return v4 ? launch_rows_g<1, 4>(L, c, q, len, w, idx, row, nrec, s) : launch_rows_g<1, 2>(L, c, q, len, w, idx, row, nrec, s);
  }
#endif
}

hipError_t BKV_SCAN_LAUNCH(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                const SeqArg& len, float* sigma, const Workspace& w, int chunk,
                                int32_t* idx, int ksel, bool skip, bool sigonly, const uint16_t* k_new,
                                const uint16_t* v_new, hipStream_t s) {
#if !BKV_QUERY_INT8 && !BKV_KEY_MXFP4 && !BKV_KEY_FP4
  if (L.query_bits == 8)
    return launch_decode_approx_q8(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
  if (L.key_format == 1)
    return launch_decode_approx_mx(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
  if (L.key_format == 2)
    return launch_decode_approx_fp4(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
#endif
#if BKV_KEY_MXFP4 || BKV_KEY_FP4  // (4-bit keys only)
  return L.v_bits == 4 ? launch_g<4, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s)
                       : launch_g<4, 2>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
#else
  const bool v4 = L.v_bits == 4;
  switch (L.k_bits) {
    case 4: return v4 ? launch_g<4, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s)
                      : launch_g<4, 2>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
    case 3: return v4 ? launch_g<3, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s)
                      : launch_g<3, 2>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
    case 2: return v4 ? launch_g<2, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s)
                      : launch_g<2, 2>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
    default: return v4 ? launch_g<1, 4>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s)
                       : launch_g<1, 2>(L, c, q, len, sigma, w, chunk, idx, ksel, skip, sigonly, k_new, v_new, s);
  }
#endif
}

}  // namespace bkv
