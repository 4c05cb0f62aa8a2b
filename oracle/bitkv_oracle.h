/*
 * bitkv_oracle.h -- CPU oracle for approximate-then-correct low-bit KV decode
 * attention.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke check and
 * the CPU-baseline leg of the benchmark may call this; the product path (the
 * HIP library and its Python binding) never does.
 *
 * The oracle is deliberately plain: scalar loops, one definition per step, no
 * blocking, fusion or reordering.  The codec (O1) runs in IEEE fp32, because
 * the stored fp16 scale/zero and the integer codes are the contract and both
 * sides must take those decisions in the same precision.  Everything after the
 * codec (scores, softmax, P.V, correction) runs in fp64.
 *
 * Sources (page titles; sections):
 *  - JetFire README, introduction: a low-bit KV cache on the GPU plus a
 *    high-precision correction of the top-k tokens ("approximate then
 *    correct").
 *  - HACK review on Pith, "What carries the argument" / "Core claim", Eq. (4):
 *    partition-wise asymmetric quantisation x ~= s*x' + m with m the partition
 *    minimum and s the step; the identity for a product of such operands.
 *  - TailorKV review on Pith, "Assumptions & free parameters": per-group
 *    quantisation with an fp16 zero point and scale; standard softmax
 *    attention and uniform quantisation definitions (its Eqs. 3 and 4).
 *  - Jet-QSparse abstract: per-KV-head selection, fp16 values with fp32
 *    accumulation in the output-forming step.
 *
 * Readings where the pages are silent:
 *  - zero point = fp16 group minimum; scale = fp16((max-min)/(2^b-1)) computed
 *    in fp32 with a correctly rounded divide; codes use the *stored* fp16
 *    scale/zero; round-to-nearest-even everywhere; a zero scale gives code 0.
 *  - groups are g consecutive channels along head_dim, per token.
 *  - query head h reads KV head h / (Hq/Hkv).
 *  - the per-KV-head selection score is the max over the query heads of the
 *    group of the approximate logit; ties go to the lower token index.
 *  - softmax scale 1/sqrt(D), no mask inside the cached tokens.
 *  - key format 2 (Jet-QSparse abstract: FP4 keys and an FP4 query-key
 *    product): the query of the approximate scores is quantised by the same
 *    MX block rule as the keys; the exact logits keep the fp16 query.
 */
#ifndef BITKV_ORACLE_H
#define BITKV_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#define ORC_MAX_D 1024 /* largest head_dim the oracle takes */

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one attention layer's cache.  D % group == 0, cap % 32 == 0. */
typedef struct {
  int32_t B, Hq, Hkv, D, kbits, vbits, group, cap;
  int32_t kfmt; /* keys: 0 = affine integer codes (O1); 1 = MXFP4 with fp16
                 * scales in the K layout, scores against the fp16 query
                 * (O1mx); 2 = MXFP4 with E8M0 scales (O1mx8, group 32) in the
                 * 32-channel-chunk layout, scores against the MXFP4 query */
} orc_shape;

/* ---- fp16 <-> fp32 (own implementation; pinned against numpy) ---- */
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f); /* round to nearest, ties to even */

/* ---- O1: quantise one group of g fp16 values to `bits`-bit codes ----
 * codes[i] in [0, 2^bits-1]; *scale16 and *zero16 are fp16 bit patterns. */
void orc_quantize_group(const uint16_t* x, int g, int bits, uint8_t* codes,
                        uint16_t* scale16, uint16_t* zero16);

/* Quantise n rows of D channels: codes[n*D] (one byte per channel) and
 * meta[n*(D/g)] = scale16 | zero16 << 16. */
void orc_quantize_rows(const uint16_t* x, int n, int D, int g, int bits,
                       uint8_t* codes, uint32_t* meta);

/* ---- O2: bit addresses of the packed layouts (bits from the unit base) ---- */
uint64_t orc_k_bitpos(int t, int c, int D, int bits);
uint64_t orc_v_bitpos(int t, int c, int D, int bits);
uint32_t orc_get_bits(const uint8_t* buf, uint64_t bitpos, int nbits);
void orc_set_bits(uint8_t* buf, uint64_t bitpos, int nbits, uint32_t value);

/* Key format 2: bit address of channel c of token t (orc_k_bitpos's role). */
uint64_t orc_k_bitpos_mx8(int t, int c, int D);

/* Buffer sizes in bytes for one whole cache. */
size_t orc_k_codes_bytes(const orc_shape* s);
size_t orc_v_codes_bytes(const orc_shape* s);
size_t orc_meta_bytes(const orc_shape* s);   /* V, and K in formats 0, 1 */
size_t orc_k_meta_bytes(const orc_shape* s); /* K in every format */
size_t orc_shadow_bytes(const orc_shape* s); /* each of K and V */

/* ---- O1+O2: append n_new tokens per sequence at positions pos[b] ----
 * k_new, v_new: [B][Hkv][n_new][D] fp16.  Writes codes, meta planes
 * [B][Hkv][D/g][cap] and the fp16 shadow [B][Hkv][cap][D]. */
void orc_pack_append(const orc_shape* s, uint8_t* k_codes, uint8_t* v_codes,
                     uint32_t* k_meta, uint32_t* v_meta, uint16_t* k_shadow,
                     uint16_t* v_shadow, const uint16_t* k_new,
                     const uint16_t* v_new, int n_new, const int32_t* pos);

/* Dequantised value of channel c of token t of unit u (fp64, exact). */
double orc_k_hat(const orc_shape* s, const uint8_t* k_codes,
                 const uint32_t* k_meta, int u, int t, int c);
double orc_v_hat(const orc_shape* s, const uint8_t* v_codes,
                 const uint32_t* v_meta, int u, int t, int c);

/* ---- O3..O5: one decode step over the cached tokens ----
 * q [B][Hq][D] fp16; len[b] tokens attended per sequence.
 * sigma [B][Hkv][cap] (fp64 selection score, first len[b] entries written);
 * idx [B][Hkv][k] int32: the selected set in ascending order, -1 padded;
 * if sel_in != NULL it is used as the selected set instead of O4 (entries
 * < 0 ignored) and idx is left untouched.
 * out [B][Hq][D]: corrected output; out_approx (S empty) and out_exact
 * (S = all tokens) are optional (NULL to skip). */
void orc_decode(const orc_shape* s, const uint8_t* k_codes,
                const uint8_t* v_codes, const uint32_t* k_meta,
                const uint32_t* v_meta, const uint16_t* k_shadow,
                const uint16_t* v_shadow, const uint16_t* q,
                const int32_t* len, int k, const int32_t* sel_in,
                double* sigma, int32_t* idx, double* out, double* out_approx,
                double* out_exact);
/* orc_decode with the approximate logits taken against the INT8 query
 * (qbits = 8, see orc_quantize_query) or against q itself (qbits = 0). */
void orc_decode_q(const orc_shape* s, const uint8_t* k_codes,
                  const uint8_t* v_codes, const uint32_t* k_meta,
                  const uint32_t* v_meta, const uint16_t* k_shadow,
                  const uint16_t* v_shadow, const uint16_t* q,
                  const int32_t* len, int k, const int32_t* sel_in, int qbits,
                  double* sigma, int32_t* idx, double* out, double* out_approx,
                  double* out_exact);

/* O1mx: one block of g fp16 values to MXFP4 (OCP Microscaling formats:
 * E2M1 elements sharing one power-of-two scale; see bitkv_oracle.c).
 * codes[i] = sign << 3 | E2M1 magnitude index; *scale16 = fp16 bits of the
 * scale (0 for an all-zero block). */
void orc_quantize_group_mx(const uint16_t* x, int g, uint8_t* codes,
                           uint16_t* scale16);
/* O1mx8: the same elements with the scale as an E8M0 byte X + 127 (no clamp;
 * an all-zero block gets 127).  Key format 2 and its query use it. */
void orc_quantize_block_mx8(const uint16_t* x, int g, uint8_t* codes,
                            uint8_t* e8);
/* the value of an E2M1 code (sign << 3 | magnitude index) */
double orc_e2m1_value(uint32_t code);

/* O1q: symmetric INT8 codes of one query row per partition of g channels
 * (codes[D], scales[D/g]); see the definition in bitkv_oracle.c. */
void orc_quantize_query(const uint16_t* q, int D, int g, int8_t* codes,
                        float* scales);

/* O4 on its own: the min(k, n) largest of sigma[0..n) by (value desc, index
 * asc), written ascending to idx[0..), rest of idx[0..k) set to -1. */
void orc_topk(const double* sigma, int n, int k, int32_t* idx);

/* O4 with a recent window of w tokens always selected: the last min(w, n)
 * tokens plus O4's min(k, n - min(w, n)) largest of the tokens before them,
 * ascending in idx[0..), the rest of idx[0..k+w) set to -1. */
void orc_topk_window(const double* sigma, int n, int k, int w, int32_t* idx);

/* O4 by blocks (Jet-QSparse abstract: the scan's scores select whole
 * 128-token blocks per KV head): block j holds tokens [j*bs, min(n, j*bs+bs))
 * and scores the maximum sigma over them; O4 picks the min(nb, ceil(n/bs))
 * best blocks (ties to the lower block), and idx[0..nb*bs) lists them in
 * ascending order, block r of the list at idx[r*bs..r*bs+bs) as its tokens
 * (-1 past n), then -1. */
void orc_topk_blocks(const double* sigma, int n, int nb, int bs, int32_t* idx);

void orc_set_threads(int n);
int orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
