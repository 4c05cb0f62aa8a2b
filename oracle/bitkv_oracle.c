/*
 * bitkv_oracle.c -- plain CPU oracle.  TEST INFRASTRUCTURE ONLY (see the
 * header).  Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no -ffast-math: the codec needs IEEE fp32 with a correctly rounded divide).
 *
 * Step names follow the method as the pages describe it:
 *   O1 quantise   asymmetric per-group uniform quantiser, x ~= s*x' + m with
 *                 m the group minimum (HACK review, Eq. (4) and "What carries
 *                 the argument"; TailorKV review, fp16 zero point and scale).
 *   O2 pack       this library's bit layouts (a storage convention, not from
 *                 the pages): K codes in 16-token blocks of (run of 8
 *                 channels, token) chunks, V codes in 32-token tiles of
 *                 dwords that each hold 8 tokens of 1 or 2 channels; both
 *                 LSB-first little-endian.
 *   O3 score      approximate logit per query head against the dequantised
 *                 keys; selection score = max over the query heads of a KV
 *                 head's group.
 *   O4 select     the top-k tokens per KV head by that score (JetFire README,
 *                 introduction: correction for top-k tokens); optionally the
 *                 newest w tokens as well, always (a recent window kept at
 *                 full precision, as the HACK review, the Jet-QSparse abstract
 *                 and the TailorKV review do).
 *   O5 correct    softmax attention where the selected tokens use exact fp16
 *                 keys/values from the shadow copy and every other token uses
 *                 the dequantised ones (JetFire README, introduction;
 *                 standard softmax attention per the TailorKV review's
 *                 "Assumptions" list).
 */
#include "bitkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ fp16 */

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp(1.0 + m / 1024.0, e - 15);
  }
  return (float)(sign ? -v : v);
}

uint16_t orc_f32_to_f16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  double a = fabs((double)f);
  if (isnan(f)) return 0x7E00;
  if (isinf(f)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: the value in units of 2^-24, rounded to nearest even
     * (rint uses the default rounding mode, round-half-even).  A result of
     * 1024 is exactly the smallest normal, whose bit pattern is also 1024. */
    double q = rint(a * ldexp(1.0, 24));
    return sign | (uint16_t)q;
  }
  int e2;
  double fr = frexp(a, &e2); /* a = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;            /* a = (2*fr) * 2^e, 2*fr in [1, 2) */
  double mant = rint((2.0 * fr - 1.0) * 1024.0);
  if (mant == 1024.0) {
    mant = 0.0;
    e += 1;
  }
  if (e > 15) return sign | 0x7C00; /* overflow to infinity */
  return sign | (uint16_t)(((e + 15) << 10) | (int)mant);
}

/* -------------------------------------------------------------- O1 codec */

void orc_quantize_group(const uint16_t* x, int g, int bits, uint8_t* codes,
                        uint16_t* scale16, uint16_t* zero16) {
  float mn = INFINITY, mx = -INFINITY;
  for (int i = 0; i < g; ++i) {
    float v = orc_f16_to_f32(x[i]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  const float qmax = (float)((1 << bits) - 1);
  const float s32 = (mx - mn) / qmax; /* fp32 subtract, correctly rounded divide */
  const uint16_t s16 = orc_f32_to_f16(s32);
  const uint16_t z16 = orc_f32_to_f16(mn); /* mn is an fp16 value: exact */
  const float s = orc_f16_to_f32(s16);
  const float z = orc_f16_to_f32(z16);
  for (int i = 0; i < g; ++i) {
    int code = 0;
    if (s != 0.0f) {
      const float v = orc_f16_to_f32(x[i]);
      const float r = rintf((v - z) / s); /* nearest, ties to even */
      code = r < 0.0f ? 0 : (r > qmax ? (int)qmax : (int)r);
    }
    codes[i] = (uint8_t)code;
  }
  *scale16 = s16;
  *zero16 = z16;
}

void orc_quantize_rows(const uint16_t* x, int n, int D, int g, int bits,
                       uint8_t* codes, uint32_t* meta) {
  const int ng = D / g;
  for (int r = 0; r < n; ++r) {
    for (int j = 0; j < ng; ++j) {
      uint16_t s16, z16;
      orc_quantize_group(x + (size_t)r * D + (size_t)j * g, g, bits,
                         codes + (size_t)r * D + (size_t)j * g, &s16, &z16);
      meta[(size_t)r * ng + j] = (uint32_t)s16 | ((uint32_t)z16 << 16);
    }
  }
}

/* O1mx: MXFP4 keys (Jet-QSparse abstract: FP4 keys; the OCP Microscaling
 * formats define the block): a block of g channels shares the scale
 * 2^X with X = floor(log2(amax)) - 2 (2 = the largest exponent of E2M1),
 * and each element is x / 2^X rounded to the nearest E2M1 magnitude
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even mantissa, larger
 * magnitudes clamped to 6) with its sign.  Readings: the scale is stored as
 * an fp16 power of two in the low half of the meta word (zero half 0), so X
 * is clamped below at -24, the smallest fp16 power of two; an all-zero block
 * has scale 0; a result of magnitude 0 carries no sign. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint32_t code) {
  const double m = kE2M1[code & 7u];
  return (code & 8u) ? -m : m;
}

/* The block's largest magnitude; *X = floor(log2(amax)) - 2 when amax > 0. */
static double mx_amax(const uint16_t* x, int g, int* X) {
  double amax = 0.0;
  for (int i = 0; i < g; ++i) {
    const double v = fabs((double)orc_f16_to_f32(x[i]));
    if (v > amax) amax = v;
  }
  if (amax > 0.0) {
    int e;
    frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
    *X = e - 1 - 2;
  }
  return amax;
}

/* Each element of the block as sign << 3 | the E2M1 index nearest to
 * |x| / 2^X (ties to the even index; above 6 the nearest is 6). */
static void mx_codes(const uint16_t* x, int g, int X, uint8_t* codes) {
  const double sc = ldexp(1.0, X);
  for (int i = 0; i < g; ++i) {
    const double v = (double)orc_f16_to_f32(x[i]);
    const double a = fabs(v) / sc;
    int best = 0;
    for (int j = 1; j < 8; ++j) { /* nearest; on a tie keep the even index */
      const double dj = fabs(a - kE2M1[j]), db = fabs(a - kE2M1[best]);
      if (dj < db || (dj == db && (j & 1) == 0)) best = j;
    }
    codes[i] = (uint8_t)(best | ((v < 0.0 && best != 0) ? 8 : 0));
  }
}

void orc_quantize_group_mx(const uint16_t* x, int g, uint8_t* codes,
                           uint16_t* scale16) {
  int X = 0;
  if (mx_amax(x, g, &X) == 0.0) {
    for (int i = 0; i < g; ++i) codes[i] = 0;
    *scale16 = 0;
    return;
  }
  if (X < -24) X = -24;
  mx_codes(x, g, X, codes);
  *scale16 = orc_f32_to_f16((float)ldexp(1.0, X));
}

/* O1mx8: the same block rule with the scale stored as its E8M0 exponent byte
 * (the OCP Microscaling formats keep the shared scale as E8M0, value
 * 2^(byte - 127)) -- the key format whose scores take the FP4 query, and that
 * query itself (Jet-QSparse abstract: FP4 keys and an FP4 query-key product).
 * Readings: X is not clamped (fp16 inputs give X in [-26, 13], inside
 * E8M0's range); an all-zero block stores X = 0 (byte 127): its codes are
 * all 0, so the scale does not matter. */
void orc_quantize_block_mx8(const uint16_t* x, int g, uint8_t* codes,
                            uint8_t* e8) {
  int X = 0;
  if (mx_amax(x, g, &X) == 0.0) {
    for (int i = 0; i < g; ++i) codes[i] = 0;
    *e8 = 127;
    return;
  }
  mx_codes(x, g, X, codes);
  *e8 = (uint8_t)(X + 127);
}

/* O1q: the query of one head quantised to INT8 per partition of g channels,
 * for scores in the HACK review's homomorphic form (Eq. (4): both operands of
 * a product quantised partition-wise, the product taken on the integer codes).
 * Reading: the query partition is symmetric, q ~= s*q' with q' in
 * [-127, 127] and no offset (zero point 0), so Eq. (4)'s term with the key
 * codes' sums vanishes:  s = amax / 127 (fp32, correctly rounded divide),
 * q' = rint(q / s) (ties to even), q' = 0 if s == 0.  The scale stays fp32:
 * the query is not stored. */
void orc_quantize_query(const uint16_t* q, int D, int g, int8_t* codes,
                        float* scales) {
  for (int p = 0; p < D / g; ++p) {
    float amax = 0.0f;
    for (int i = 0; i < g; ++i) {
      const float v = fabsf(orc_f16_to_f32(q[p * g + i]));
      if (v > amax) amax = v;
    }
    const float s = amax / 127.0f;
    for (int i = 0; i < g; ++i) {
      int code = 0;
      if (s != 0.0f) {
        const float r = rintf(orc_f16_to_f32(q[p * g + i]) / s);
        code = r < -127.0f ? -127 : (r > 127.0f ? 127 : (int)r);
      }
      codes[p * g + i] = (int8_t)code;
    }
    scales[p] = s;
  }
}

/* -------------------------------------------------------------- O2 layout */

/* K: blocks of 16 tokens.  Channel c has group g = c / 32, eighth
 * e = (c mod 32) / 8 (which 8-channel run of its group) and offset j = c mod 8.
 * A block is 64 chunks in the order (e, token mod 16); a chunk is the D/32
 * group fields of one (token, e) in group order, and a field is the 8 codes
 * of that run, code j at bits [j*bits, j*bits+bits).  Bits are counted
 * LSB-first through little-endian bytes, so with 3 bits a 24-bit field may
 * straddle 32-bit words. */
uint64_t orc_k_bitpos(int t, int c, int D, int bits) {
  const int ng = D / 32;
  const int g = c / 32, e = (c % 32) / 8, j = c % 8;
  const uint64_t field_bits = 8u * (uint64_t)bits;
  const uint64_t chunk_bits = (uint64_t)ng * field_bits;
  const uint64_t chunk = (uint64_t)e * 16u + (uint64_t)(t % 16);
  return (uint64_t)(t / 16) * 16u * (uint64_t)D * bits + chunk * chunk_bits +
         (uint64_t)g * field_bits + (uint64_t)j * bits;
}

/* K in key format 2 (4-bit E2M1 codes): blocks of 16 tokens, each
 * (D/32)*16 chunks of 16 bytes; chunk 16*g + (t mod 16) holds the 32 codes
 * of channels 32g .. 32g+31 of token t, channel 32g + j at bits 4j..4j+3
 * (two codes a byte, the lower channel in the low half). */
uint64_t orc_k_bitpos_mx8(int t, int c, int D) {
  const uint64_t chunk = 16u * (uint64_t)(c / 32) + (uint64_t)(t % 16);
  return (uint64_t)(t / 16) * 16u * (uint64_t)D * 4u + chunk * 128u + 4u * (uint64_t)(c % 32);
}

/* V (bits 2 or 4): tiles of 32 tokens.  Token r of the tile (r = t mod 32)
 * lies in quarter q = (r mod 16) / 4 at slot j = 4*(r / 16) + r mod 4.
 * Channel c belongs to owner l = 16*q + c mod 16 as column n = c / 16.  A
 * 32-bit dword holds 4/bits columns of one owner: column n is in dword
 * d = n / (4/bits) at sub-position s = n mod (4/bits), and its slot j sits at
 * bit 16*(j / 4) + 4*bits*s + bits*(j mod 4) of that dword (slots 0..3 in the
 * low half, 4..7 in the high half).  The tile stores dword d of owner l at
 * index 256*(d / 4) + 4*l + d mod 4: 16-byte pieces, piece-major. */
uint64_t orc_v_bitpos(int t, int c, int D, int bits) {
  const int tile = t / 32;
  const int r = t % 32;
  const int q = (r % 16) / 4;
  const int j = 4 * (r / 16) + (r % 4);
  const int l = 16 * q + c % 16;
  const int n = c / 16;
  const int cpd = 4 / bits;
  const int d = n / cpd, sub = n % cpd;
  const uint64_t dw = 256u * (uint64_t)(d / 4) + 4u * (uint64_t)l + (uint64_t)(d % 4);
  const uint64_t bit = 16u * (uint64_t)(j / 4) + 4u * (uint64_t)bits * sub + (uint64_t)bits * (j % 4);
  return (uint64_t)tile * 32u * (uint64_t)D * bits + dw * 32u + bit;
}

uint32_t orc_get_bits(const uint8_t* buf, uint64_t bitpos, int nbits) {
  uint32_t v = 0;
  for (int i = 0; i < nbits; ++i) {
    const uint64_t p = bitpos + (uint64_t)i;
    const uint32_t bit = (buf[p / 8] >> (p % 8)) & 1u;
    v |= bit << i;
  }
  return v;
}

void orc_set_bits(uint8_t* buf, uint64_t bitpos, int nbits, uint32_t value) {
  for (int i = 0; i < nbits; ++i) {
    const uint64_t p = bitpos + (uint64_t)i;
    const uint8_t mask = (uint8_t)(1u << (p % 8));
    if ((value >> i) & 1u)
      buf[p / 8] |= mask;
    else
      buf[p / 8] &= (uint8_t)~mask;
  }
}

static size_t units_of(const orc_shape* s) { return (size_t)s->B * s->Hkv; }
static size_t k_unit_bytes(const orc_shape* s) {
  return (size_t)s->cap * s->D * s->kbits / 8;
}
static size_t v_unit_bytes(const orc_shape* s) {
  return (size_t)s->cap * s->D * s->vbits / 8;
}
size_t orc_k_codes_bytes(const orc_shape* s) { return units_of(s) * k_unit_bytes(s); }
size_t orc_v_codes_bytes(const orc_shape* s) { return units_of(s) * v_unit_bytes(s); }
size_t orc_meta_bytes(const orc_shape* s) {
  return units_of(s) * (size_t)(s->D / s->group) * s->cap * sizeof(uint32_t);
}
/* Key format 2 keeps one E8M0 byte per (token, 32-channel block),
 * [B][Hkv][cap][D/32]; the other formats use the meta planes. */
size_t orc_k_meta_bytes(const orc_shape* s) {
  if (s->kfmt == 2) return units_of(s) * (size_t)s->cap * (size_t)(s->D / 32);
  return orc_meta_bytes(s);
}
static size_t k_scale_index(const orc_shape* s, int u, int t, int blk) {
  return ((size_t)u * s->cap + t) * (size_t)(s->D / 32) + blk;
}
static uint64_t k_code_bitpos(const orc_shape* s, int t, int c) {
  return s->kfmt == 2 ? orc_k_bitpos_mx8(t, c, s->D) : orc_k_bitpos(t, c, s->D, s->kbits);
}
size_t orc_shadow_bytes(const orc_shape* s) {
  return units_of(s) * (size_t)s->cap * s->D * sizeof(uint16_t);
}

static size_t meta_index(const orc_shape* s, int u, int grp, int t) {
  return ((size_t)u * (s->D / s->group) + grp) * (size_t)s->cap + t;
}

void orc_pack_append(const orc_shape* s, uint8_t* k_codes, uint8_t* v_codes,
                     uint32_t* k_meta, uint32_t* v_meta, uint16_t* k_shadow,
                     uint16_t* v_shadow, const uint16_t* k_new,
                     const uint16_t* v_new, int n_new, const int32_t* pos) {
  const int D = s->D, g = s->group, ng = s->D / s->group;
  uint8_t* codes = (uint8_t*)malloc((size_t)D);
  uint32_t* meta = (uint32_t*)malloc((size_t)ng * sizeof(uint32_t));
  for (int b = 0; b < s->B; ++b) {
    for (int kvh = 0; kvh < s->Hkv; ++kvh) {
      const int u = b * s->Hkv + kvh;
      for (int j = 0; j < n_new; ++j) {
        const int t = pos[b] + j;
        const size_t src = (((size_t)u * n_new) + j) * D;
        /* keys */
        if (s->kfmt == 2) {
          for (int blk = 0; blk < D / 32; ++blk)
            orc_quantize_block_mx8(k_new + src + (size_t)blk * 32, 32, codes + (size_t)blk * 32,
                                   (uint8_t*)k_meta + k_scale_index(s, u, t, blk));
        } else if (s->kfmt == 1) {
          for (int grp = 0; grp < ng; ++grp) {
            uint16_t s16;
            orc_quantize_group_mx(k_new + src + (size_t)grp * g, g, codes + (size_t)grp * g, &s16);
            meta[grp] = s16;
          }
        } else {
          orc_quantize_rows(k_new + src, 1, D, g, s->kbits, codes, meta);
        }
        for (int c = 0; c < D; ++c)
          orc_set_bits(k_codes + (size_t)u * k_unit_bytes(s), k_code_bitpos(s, t, c), s->kbits, codes[c]);
        if (s->kfmt != 2)
          for (int grp = 0; grp < ng; ++grp) k_meta[meta_index(s, u, grp, t)] = meta[grp];
        memcpy(k_shadow + ((size_t)u * s->cap + t) * D, k_new + src, (size_t)D * 2);
        /* values */
        orc_quantize_rows(v_new + src, 1, D, g, s->vbits, codes, meta);
        for (int c = 0; c < D; ++c)
          orc_set_bits(v_codes + (size_t)u * v_unit_bytes(s),
                       orc_v_bitpos(t, c, D, s->vbits), s->vbits, codes[c]);
        for (int grp = 0; grp < ng; ++grp) v_meta[meta_index(s, u, grp, t)] = meta[grp];
        memcpy(v_shadow + ((size_t)u * s->cap + t) * D, v_new + src, (size_t)D * 2);
      }
    }
  }
  free(codes);
  free(meta);
}

/* x_hat = s * code + z, evaluated in fp64 (exact for fp16 s, z and small
 * integer codes). */
static double dequant(uint32_t meta, uint32_t code) {
  const double sc = orc_f16_to_f32((uint16_t)(meta & 0xFFFFu));
  const double z = orc_f16_to_f32((uint16_t)(meta >> 16));
  return sc * (double)code + z;
}

double orc_k_hat(const orc_shape* s, const uint8_t* k_codes,
                 const uint32_t* k_meta, int u, int t, int c) {
  const uint32_t code = orc_get_bits(k_codes + (size_t)u * k_unit_bytes(s), k_code_bitpos(s, t, c), s->kbits);
  if (s->kfmt == 2) /* the E2M1 value times 2^(E8M0 byte - 127) */
    return ldexp(orc_e2m1_value(code), (int)((const uint8_t*)k_meta)[k_scale_index(s, u, t, c / 32)] - 127);
  const uint32_t meta = k_meta[meta_index(s, u, c / s->group, t)];
  if (s->kfmt == 1) /* MXFP4: the E2M1 value times the block's power of two */
    return orc_e2m1_value(code) * (double)orc_f16_to_f32((uint16_t)(meta & 0xFFFFu));
  return dequant(meta, code);
}

double orc_v_hat(const orc_shape* s, const uint8_t* v_codes,
                 const uint32_t* v_meta, int u, int t, int c) {
  const uint32_t code = orc_get_bits(v_codes + (size_t)u * v_unit_bytes(s),
                                     orc_v_bitpos(t, c, s->D, s->vbits), s->vbits);
  return dequant(v_meta[meta_index(s, u, c / s->group, t)], code);
}

/* -------------------------------------------------------------- O4 top-k */

typedef struct {
  double v;
  int32_t t;
} scored;

static int by_score_desc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->t > y->t) - (x->t < y->t); /* equal scores: lower index first */
}

static int by_int_asc(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

void orc_topk(const double* sigma, int n, int k, int32_t* idx) {
  const int kk = k < n ? k : n;
  scored* all = (scored*)malloc((size_t)(n > 0 ? n : 1) * sizeof(scored));
  for (int t = 0; t < n; ++t) {
    all[t].v = sigma[t];
    all[t].t = t;
  }
  qsort(all, (size_t)n, sizeof(scored), by_score_desc);
  for (int i = 0; i < kk; ++i) idx[i] = all[i].t;
  qsort(idx, (size_t)kk, sizeof(int32_t), by_int_asc);
  for (int i = kk; i < k; ++i) idx[i] = -1;
  free(all);
}

/* O4 with an exact recent window (the HACK review keeps the newest block in
 * fp16, the Jet-QSparse abstract keeps recent pages in BF16, TailorKV keeps
 * local tokens at full precision): the last min(w, n) tokens are always in
 * the set, and O4 picks k more among the tokens before them. */
void orc_topk_window(const double* sigma, int n, int k, int w, int32_t* idx) {
  const int nw = w < n ? w : n;
  const int n0 = n - nw;
  const int kk = k < n0 ? k : n0;
  orc_topk(sigma, n0, k, idx); /* idx[0..kk) ascending, idx[kk..k) = -1 */
  for (int i = 0; i < nw; ++i) idx[kk + i] = n0 + i;
  for (int i = kk + nw; i < k + w; ++i) idx[i] = -1;
}

/* O4 over blocks of bs tokens scored by their largest sigma: the top-k of the
 * block scores, each chosen block then expanded to its tokens. */
void orc_topk_blocks(const double* sigma, int n, int nb, int bs, int32_t* idx) {
  const int nblk = (n + bs - 1) / bs;
  double* score = (double*)malloc((size_t)(nblk > 0 ? nblk : 1) * sizeof(double));
  int32_t* chosen = (int32_t*)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(int32_t));
  for (int j = 0; j < nblk; ++j) {
    double m = -INFINITY;
    for (int t = j * bs; t < n && t < (j + 1) * bs; ++t)
      if (sigma[t] > m) m = sigma[t];
    score[j] = m;
  }
  orc_topk(score, nblk, nb, chosen); /* ascending block indices, then -1 */
  for (int r = 0; r < nb; ++r)
    for (int x = 0; x < bs; ++x) {
      const long long t = (long long)chosen[r] * bs + x;
      idx[(size_t)r * bs + x] = (chosen[r] >= 0 && t < n) ? (int32_t)t : -1;
    }
  free(score);
  free(chosen);
}

/* ------------------------------------------------------- O3 + O5 (fp64) */

/* out[h][0..D) = sum_t e^{lambda_t - m} nu_t / sum_t e^{lambda_t - m} for one
 * query head, where token t uses the exact logit/value if in_s[t] and the
 * approximate ones otherwise.  shat: approximate logits of this head. */
static void attend_head(const orc_shape* s, int u, int n, const double* shat,
                        const double* sexact, const uint8_t* in_s,
                        const uint8_t* v_codes, const uint32_t* v_meta,
                        const uint16_t* v_shadow, double* out) {
  const int D = s->D;
  if (n == 0) {
    for (int c = 0; c < D; ++c) out[c] = 0.0;
    return;
  }
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    const double lam = in_s[t] ? sexact[t] : shat[t];
    if (lam > m) m = lam;
  }
  double den = 0.0;
  for (int c = 0; c < D; ++c) out[c] = 0.0;
  for (int t = 0; t < n; ++t) {
    const double lam = in_s[t] ? sexact[t] : shat[t];
    const double p = exp(lam - m);
    den += p;
    for (int c = 0; c < D; ++c) {
      const double nu =
          in_s[t] ? (double)orc_f16_to_f32(v_shadow[((size_t)u * s->cap + t) * D + c])
                  : orc_v_hat(s, v_codes, v_meta, u, t, c);
      out[c] += p * nu;
    }
  }
  for (int c = 0; c < D; ++c) out[c] /= den;
}

void orc_decode(const orc_shape* s, const uint8_t* k_codes,
                const uint8_t* v_codes, const uint32_t* k_meta,
                const uint32_t* v_meta, const uint16_t* k_shadow,
                const uint16_t* v_shadow, const uint16_t* q,
                const int32_t* len, int k, const int32_t* sel_in,
                double* sigma, int32_t* idx, double* out, double* out_approx,
                double* out_exact) {
  orc_decode_q(s, k_codes, v_codes, k_meta, v_meta, k_shadow, v_shadow, q, len,
               k, sel_in, 0, sigma, idx, out, out_approx, out_exact);
}

/* qbits = 8: the approximate logits (O3) use the dequantised INT8 query
 * s*q' (O1q) in place of q; key format 2: they use the MXFP4 query (O1mx8 on
 * each 32-channel block of each query head), so each score is the FP4 query
 * times the FP4 keys.  The exact logits of the correction keep q. */
void orc_decode_q(const orc_shape* s, const uint8_t* k_codes,
                  const uint8_t* v_codes, const uint32_t* k_meta,
                  const uint32_t* v_meta, const uint16_t* k_shadow,
                  const uint16_t* v_shadow, const uint16_t* q,
                  const int32_t* len, int k, const int32_t* sel_in, int qbits,
                  double* sigma, int32_t* idx, double* out, double* out_approx,
                  double* out_exact) {
  const int G = s->Hq / s->Hkv;
  const int D = s->D;
  const double sm = 1.0 / sqrt((double)D);
  const int U = s->B * s->Hkv;

#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < U; ++u) {
    const int b = u / s->Hkv;
    const int kvh = u % s->Hkv;
    const int n = len[b];
    const int nn = n > 0 ? n : 1;
    double* shat = (double*)malloc((size_t)G * nn * sizeof(double));
    double* sexact = (double*)malloc((size_t)G * nn * sizeof(double));
    uint8_t* in_s = (uint8_t*)calloc((size_t)nn, 1);
    uint8_t* none = (uint8_t*)calloc((size_t)nn, 1);
    uint8_t* all = (uint8_t*)malloc((size_t)nn);
    memset(all, 1, (size_t)nn);
    double* sig = sigma + (size_t)u * s->cap;

    /* the query of the approximate logits: q, its INT8 form s*q', or (key
     * format 2) its MXFP4 form, the E2M1 values times each block's 2^X */
    double* qa = (double*)malloc((size_t)G * D * sizeof(double));
    for (int i = 0; i < G; ++i) {
      const uint16_t* qh = q + ((size_t)b * s->Hq + (size_t)kvh * G + i) * D;
      if (s->kfmt == 2) {
        for (int blk = 0; blk < D / 32; ++blk) {
          uint8_t qc[32], e8;
          orc_quantize_block_mx8(qh + (size_t)blk * 32, 32, qc, &e8);
          for (int j = 0; j < 32; ++j)
            qa[(size_t)i * D + blk * 32 + j] = ldexp(orc_e2m1_value(qc[j]), (int)e8 - 127);
        }
      } else if (qbits == 8) {
        int8_t qc[ORC_MAX_D];
        float qs[ORC_MAX_D];
        orc_quantize_query(qh, D, s->group, qc, qs);
        for (int c = 0; c < D; ++c) qa[(size_t)i * D + c] = (double)qs[c / s->group] * qc[c];
      } else {
        for (int c = 0; c < D; ++c) qa[(size_t)i * D + c] = orc_f16_to_f32(qh[c]);
      }
    }

    /* O3: approximate logits and the selection score. */
    for (int t = 0; t < n; ++t) {
      double best = -INFINITY;
      for (int i = 0; i < G; ++i) {
        const uint16_t* qh = q + ((size_t)b * s->Hq + (size_t)kvh * G + i) * D;
        double acc = 0.0, ex = 0.0;
        for (int c = 0; c < D; ++c) {
          const double qc = orc_f16_to_f32(qh[c]);
          acc += qa[(size_t)i * D + c] * orc_k_hat(s, k_codes, k_meta, u, t, c);
          ex += qc * (double)orc_f16_to_f32(k_shadow[((size_t)u * s->cap + t) * D + c]);
        }
        shat[(size_t)i * nn + t] = sm * acc;
        sexact[(size_t)i * nn + t] = sm * ex;
        if (sm * acc > best) best = sm * acc;
      }
      sig[t] = best;
    }

    /* O4: the selected set. */
    int32_t* my_idx = idx + (size_t)u * (k > 0 ? k : 0);
    if (sel_in) {
      const int32_t* si = sel_in + (size_t)u * (k > 0 ? k : 0);
      for (int i = 0; i < k; ++i)
        if (si[i] >= 0 && si[i] < n) in_s[si[i]] = 1;
    } else if (k > 0) {
      orc_topk(sig, n, k, my_idx);
      for (int i = 0; i < k; ++i)
        if (my_idx[i] >= 0) in_s[my_idx[i]] = 1;
    }

    /* O5: per query head of the group. */
    for (int i = 0; i < G; ++i) {
      const size_t h = (size_t)b * s->Hq + (size_t)kvh * G + i;
      const double* sh = shat + (size_t)i * nn;
      const double* se = sexact + (size_t)i * nn;
      attend_head(s, u, n, sh, se, in_s, v_codes, v_meta, v_shadow, out + h * D);
      if (out_approx)
        attend_head(s, u, n, sh, se, none, v_codes, v_meta, v_shadow, out_approx + h * D);
      if (out_exact)
        attend_head(s, u, n, sh, se, all, v_codes, v_meta, v_shadow, out_exact + h * D);
    }
    free(qa);
    free(shat);
    free(sexact);
    free(in_s);
    free(none);
    free(all);
  }
}

void orc_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
