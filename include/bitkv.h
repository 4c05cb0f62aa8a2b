/*
 * bitkv.h -- C ABI of libbitkv.so: approximate-then-correct low-bit KV decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method (JetFire README, introduction; title "Approximate-then-Correct
 * Attention on Hybrid Memory"): keep the KV cache in low-bit form, compute
 * attention approximately over it, pick the top-k tokens, and correct those
 * tokens with exact high-precision keys and values.  The quantiser is the
 * asymmetric per-group one of the HACK review on Pith (Eq. (4), "What carries
 * the argument": x ~= s*x' + m, m the group minimum) with an fp16 scale and
 * zero point per group (TailorKV review on Pith, "Assumptions & free
 * parameters").  Top-k is taken per KV head (Jet-QSparse abstract: the
 * selection budget is per KV head).
 *
 * A decode step is a few of these calls on one stream (the plainest: append,
 * approximate pass, top-k, correction):
 *   kv_pack_append       quantise + pack the new token(s), write the shadow
 *   qattn_decode_approx  approximate scores, selection score, split softmax.V
 *   qattn_decode_select  the same and topk_select, in one launch where it fits
 *   qattn_decode_step    kv_pack_append of one token + qattn_decode_select, one launch
 *   qattn_decode_fused   the whole step (append, scan, top-k, correction) in one launch
 *   topk_select          top-k tokens per KV head by the selection score
 *   topk_select_window   the same, plus the newest tokens always selected
 *   topk_select_blocks   or whole blocks of tokens by their best score
 *   qattn_correct        merge the splits, replace the top-k tokens' logits
 *                        and values by exact ones, renormalise
 *   qattn_correct_blocks the same for block rows, over contiguous tiles
 *   qattn_score_select   sigma and the top-k rows only (no softmax state)
 *   qattn_decode_unselected, qattn_correct_unselected
 *                        the approximate pass over the unselected tokens only,
 *                        then the exact terms merged in (no subtraction)
 *   qattn_exact_host     (host) exact states of the selected tokens from a
 *                        host copy of the shadow rows, for
 *   qattn_correct_hybrid qattn_correct with those exact states
 *   qattn_hybrid_layers  (host schedule) the hybrid step over several layers,
 *                        host passes overlapping GPU work
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers unless the name ends in _host.
 *    Shadow pointers may also be device-visible pinned host memory (see
 *    bkv_cache).  The caller owns every buffer; the library never allocates,
 *    frees or synchronises, and keeps no state between calls (the one
 *    host-only computation, qattn_exact_host, uses OpenMP's thread pool;
 *    qattn_hybrid_layers waits on events of its own; qattn_decode_fused_noalloc
 *    uses an array the library holds; qattn_correct_blocks forks onto a
 *    stream of the library's and joins back).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work; results are ready when the stream is.
 *  - Errors: every call validates its arguments on the host before any launch
 *    and returns a status; it never aborts, throws or prints.  On any status
 *    other than BKV_OK nothing was enqueued, except BKV_E_HIP, which reports
 *    a failed launch (hipGetLastError) of one of the call's kernels.
 *  - Supported shapes: head_dim 128, group 32 or 64, k_bits in {1, 2, 3, 4},
 *    v_bits in {2, 4}, n_q_heads / n_kv_heads in {4, 8}, capacity a positive
 *    multiple of 32, batch in [1, 256], query_bits 0 or 8, key_format 0, 1
 *    or 2 (1 and 2: k_bits 4, group 32, query_bits 0).  Others return
 *    BKV_E_UNSUPPORTED or BKV_E_SHAPE.
 *  - Query head h attends with KV head h / (n_q_heads / n_kv_heads).
 *  - Softmax scale 1/sqrt(head_dim); no mask inside the cached tokens.
 *  - Inputs must be finite fp16 values.
 */
#ifndef BITKV_H
#define BITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BKV_OK = 0,
  BKV_E_NULL = 1,        /* a required pointer is NULL                       */
  BKV_E_SHAPE = 2,       /* inconsistent sizes (e.g. Hq % Hkv, capacity % 32) */
  BKV_E_UNSUPPORTED = 3, /* valid but not built (bits, head_dim, group, G)     */
  BKV_E_CAPACITY = 4,    /* a position or length outside [0, capacity]         */
  BKV_E_WORKSPACE = 5,   /* workspace smaller than bkv_workspace_bytes         */
  BKV_E_HIP = 6,         /* a kernel launch failed                             */
  BKV_E_ARG = 7          /* other invalid scalar argument (k < 0, n_new < 0)   */
} bkv_status;

/* Shape of one attention layer's cache. */
typedef struct {
  int32_t batch;      /* B                                                  */
  int32_t n_q_heads;  /* Hq                                                 */
  int32_t n_kv_heads; /* Hkv; units are the B*Hkv (batch, KV head) pairs    */
  int32_t head_dim;   /* D (128)                                            */
  int32_t k_bits;     /* bits per key code (1, 2, 3 or 4)                   */
  int32_t v_bits;     /* bits per value code (2 or 4)                       */
  int32_t group;      /* channels per quantisation group along D (32, 64)   */
  int32_t capacity;   /* token slots per unit, multiple of 32               */
  int32_t query_bits; /* query of the approximate scores: 0 = the fp16 query
                       * as given; 8 = that query quantised per group to
                       * symmetric INT8 (HACK review on Pith, Eq. (4): both
                       * operands of Q.K^T quantised, the product taken on the
                       * integer codes; here s = amax/127 in fp32,
                       * q' = rint(q/s) in [-127, 127], so the term with the
                       * key code sums is zero).  The exact logits of the
                       * correction always use the fp16 query.              */
  int32_t key_format; /* key codes: 0 = affine (s * code + z per group, k_bits
                       * bits); 1 = MXFP4 (Jet-QSparse abstract: FP4 keys;
                       * OCP Microscaling block format): each group of 32
                       * shares a power-of-two scale 2^X, X = floor(log2
                       * amax) - 2 (clamped at -24), stored as fp16 in the
                       * meta word's low half (high half 0), and a code is
                       * sign << 3 | the E2M1 magnitude index (0, 0.5, 1,
                       * 1.5, 2, 3, 4, 6) of x / 2^X, nearest, ties to the
                       * even index, clamped at 6.  Needs k_bits 4, group 32,
                       * query_bits 0; the key bit layout is that of K4.  The
                       * approximate scores take the fp16 query (a variant
                       * kept beside format 2).
                       * 2 = MXFP4 keys scored against an MXFP4 query
                       * (Jet-QSparse abstract: FP4 keys and a native FP4
                       * query-key product): keys and, inside the scan, each
                       * 32-channel block of each query head get the same
                       * rule as format 1 with the scale kept as the E8M0
                       * byte X + 127 (X unclamped; 127 for an all-zero
                       * block), and the scores are the FP4 x FP4 products
                       * on gfx950's scaled FP4 MFMA.  Layouts below.  The
                       * exact logits of the correction keep the fp16 query.
                       * Needs k_bits 4, group 32, query_bits 0.            */
} bkv_layout;

/*
 * The cache of one layer.  Unit u = b * Hkv + kvh is the outermost index of
 * every buffer.  Sizes come from bkv_cache_bytes.  Zero-fill the code buffers
 * before the first append: appends read-modify-write the shared V words.
 *
 *  k_codes  [B][Hkv][capacity/16][64][4*k_bits] bytes: blocks of 16 tokens.
 *           Channel c = 32g + 8e + j (group g, eighth e, offset j).  Chunk
 *           (e, r) of a block, at index 16e + r, holds the codes of token r
 *           of the block for channels 32g + 8e + j in the order (g, j),
 *           k_bits each, LSB-first little-endian (with 3 bits a code can
 *           straddle a 32-bit word).  16-byte aligned.
 *  v_codes  [B][Hkv][capacity/32][128*v_bits] uint32: tiles of 32 tokens.
 *           Token r of the tile is in quarter q = (r mod 16)/4 at slot
 *           j = 4*(r/16) + r mod 4; channel c has owner l = 16q + c mod 16
 *           and column n = c/16.  With m = 4/v_bits columns per dword,
 *           column n is in dword d = n/m at sub-position s = n mod m, and
 *           slot j is at bit 16*(j/4) + 4*v_bits*s + v_bits*(j mod 4) of it.
 *           Dword d of owner l is dword 256*(d/4) + 4l + d mod 4 of the
 *           tile.  16-byte aligned.
 *  k_meta,  [B][Hkv][D/group][capacity] uint32: fp16 scale in the low half,
 *  v_meta   fp16 zero point (group minimum) in the high half.
 *  Key format 2 instead:
 *  k_codes  [B][Hkv][capacity/16][64][16] bytes: chunk 16g + r of a block
 *           holds the 32 codes of channels 32g..32g+31 of token r of the
 *           block, channel 32g + j in nibble j (low nibble first).
 *  k_meta   [B][Hkv][capacity] uint32: byte g (bits 8g..8g+7) of token t's
 *           word is the E8M0 scale of its channels 32g..32g+31 (only these
 *           B*Hkv*capacity words are used: bkv_k_meta_bytes gives the size;
 *           a buffer of meta_bytes_each is also large enough).
 *  k_shadow,[B][Hkv][capacity][D] fp16: the exact input rows.  Device memory,
 *  v_shadow or pinned host memory the device can address (e.g. hipHostMalloc
 *           with default flags): qattn_correct then gathers the selected
 *           rows across PCIe.
 */
typedef struct {
  void* k_codes;
  void* v_codes;
  uint32_t* k_meta;
  uint32_t* v_meta;
  uint16_t* k_shadow;
  uint16_t* v_shadow;
} bkv_cache;

/* Byte sizes of the cache buffers for `layout`.  Host only. */
bkv_status bkv_cache_bytes(const bkv_layout* layout, size_t* k_codes_bytes,
                           size_t* v_codes_bytes, size_t* meta_bytes_each,
                           size_t* shadow_bytes_each);

/* Bytes k_meta needs for `layout`: meta_bytes_each for key formats 0 and 1,
 * B*Hkv*capacity*4 (one word of four E8M0 bytes per token) for key format 2.
 * Host only. */
bkv_status bkv_k_meta_bytes(const bkv_layout* layout, size_t* bytes);

/* Workspace bytes that cover qattn_decode_approx, topk_select and
 * qattn_correct (and every variant below) for every step whose longest
 * sequence has at most max_len tokens and whose row length is k.  Host only.  One workspace serves the
 * three calls of a step (the scan's split states, the top-k candidates and
 * arrival counters and the correction's chunk states live in it).  Zero-fill
 * it once after allocating it; every call leaves the counters at zero again.
 * They sit at the start, one per (batch, KV head): zero-fill again before a
 * call whose layout has more batch * n_kv_heads than the calls before it on
 * this workspace.  Calls that may run concurrently (on different streams)
 * need separate workspaces. */
bkv_status bkv_workspace_bytes(const bkv_layout* layout, int32_t max_len,
                               int32_t k, size_t* bytes);

/*
 * kv_pack_append -- quantise and store n_new tokens per sequence (HACK review
 * on Pith, Eq. (4) and "What carries the argument": per-partition asymmetric
 * quantisation x ~= s*x' + m with m the partition minimum; TailorKV review on
 * Pith, "Assumptions & free parameters": fp16 zero point and scale per group;
 * JetFire README, introduction: the exact copy kept beside the low-bit cache).
 * For each (b, kvh) and j < n_new the token k_new/v_new[b][kvh][j][0..D)
 * (fp16, device) goes to slot t = pos_host[b] + j: per group of 32 channels
 * the fp16 zero z = min, scale s = fp16((max - min) / (2^bits - 1)) computed
 * in fp32 with a correctly rounded divide, and codes
 * clamp(rint((x - z) / s), 0, 2^bits - 1) from the stored fp16 s and z (0 when
 * s is 0), round to nearest even throughout; then the bits, the meta words and
 * the verbatim shadow row.
 * Errors: BKV_E_CAPACITY unless 0 <= pos_host[b] and pos_host[b] + n_new <=
 * capacity; BKV_E_ARG if n_new < 0 (n_new == 0 enqueues nothing).
 */
bkv_status kv_pack_append(const bkv_layout* layout, const bkv_cache* cache,
                          const uint16_t* k_new, const uint16_t* v_new,
                          int32_t n_new, const int32_t* pos_host, void* stream);

/*
 * qattn_decode_approx -- the approximate pass over the packed cache.
 * q [B][Hq][D] fp16 (device).  Sequence b attends to its first len_host[b]
 * tokens.  For every query head h and token t the approximate logit is
 *   s_hat[h][t] = (1/sqrt(D)) * sum_c q[h][c] * (s * code + z),
 * evaluated as sum over groups of s * (q . codes) + z * sum(q) (HACK review,
 * Eq. (4), with an unquantised query).  Writes
 *   sigma [B][Hkv][capacity] fp32: sigma[t] = max over the KV head's query
 *         heads of s_hat[h][t] for t < len (slots up to the next multiple of
 *         32 get -inf; others untouched);
 *   ws:   per (b, h, split) the softmax state (running max in log2 units,
 *         denominator, unnormalised sum of p * V_hat) of its token range.
 * Errors: BKV_E_CAPACITY if some len_host[b] is outside [0, capacity];
 * BKV_E_WORKSPACE if ws_bytes is too small (bkv_workspace_bytes).
 */
bkv_status qattn_decode_approx(const bkv_layout* layout, const bkv_cache* cache,
                               const uint16_t* q, const int32_t* len_host,
                               float* sigma, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * qattn_decode_select -- qattn_decode_approx followed by topk_select with the
 * same layout, cache, q, lengths, k and workspace, with identical results
 * (sigma, the split states in ws and idx [B][Hkv][k]).  The selection can run
 * inside the scan's launch: every scan workgroup keeps its token range's
 * sigma on chip, leaves the range's top-min(k, len) candidates in ws, and
 * the last workgroup of each (b, kvh) to finish merges them.  That needs
 * each range at most 16384 tokens and ranges per (b, kvh) times k at most
 * 8192.  mode: 0 = automatic (in the scan's launch when also each range is
 * at least 8192 tokens long, where it is faster), 1 = in the scan's launch
 * whenever possible, 2 = always the two launches.  k == 0 is
 * qattn_decode_approx (idx may then be NULL).  Size ws with
 * bkv_workspace_bytes(layout, max_len, k).
 * Errors: BKV_E_ARG for a mode outside 0..2; otherwise as
 * qattn_decode_approx and topk_select.
 */
bkv_status qattn_decode_select(const bkv_layout* layout, const bkv_cache* cache,
                               const uint16_t* q, const int32_t* len_host,
                               int32_t k, float* sigma, int32_t* idx, void* ws,
                               size_t ws_bytes, int32_t mode, void* stream);

/*
 * qattn_decode_step -- kv_pack_append of one token per sequence at position
 * len_host[b] - 1 (k_new, v_new [B][Hkv][D] fp16, device) followed by
 * qattn_decode_select over len_host[b] tokens, in the scan's launch: the scan
 * workgroup whose token range holds that position quantises and stores the
 * token (codes, meta, shadow row; the same bits kv_pack_append writes)
 * before it reads the cache.  Results identical to the two calls; mode as in
 * qattn_decode_select.
 * Errors: BKV_E_CAPACITY if some len_host[b] < 1 or > capacity; otherwise as
 * qattn_decode_select.
 */
bkv_status qattn_decode_step(const bkv_layout* layout, const bkv_cache* cache,
                             const uint16_t* k_new, const uint16_t* v_new,
                             const uint16_t* q, const int32_t* len_host, int32_t k,
                             float* sigma, int32_t* idx, void* ws, size_t ws_bytes,
                             int32_t mode, void* stream);

/* Host only: *in_scan = 1 if qattn_decode_select with this layout, longest
 * length max_len, k and mode selects inside the scan's launch, else 0. */
bkv_status bkv_select_in_scan(const bkv_layout* layout, int32_t max_len, int32_t k,
                              int32_t mode, int32_t* in_scan);

/*
 * topk_select -- per (b, kvh): the min(k, len) tokens with the largest sigma,
 * ties broken towards the lower index (JetFire README, introduction: top-k
 * tokens get the high-precision correction; Jet-QSparse abstract: the budget
 * is per KV head).  idx [B][Hkv][k] int32 (device) receives the selected token
 * indices in ascending order, -1 after the min(k, len)-th entry.  Uses the
 * top-k scratch region of ws.  k == 0 enqueues nothing.
 * Errors: BKV_E_ARG if k < 0; BKV_E_CAPACITY for a bad length;
 * BKV_E_WORKSPACE if ws is too small.
 */
bkv_status topk_select(const bkv_layout* layout, const float* sigma,
                       const int32_t* len_host, int32_t k, int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * topk_select_window -- topk_select with a recent window: per (b, kvh) the
 * newest nw = min(window, len) tokens are always selected (HACK review and
 * TailorKV review: the most recent tokens stay at full precision; Jet-QSparse
 * abstract: the top-k budget is per KV head) and the top-k runs over the
 * first n = len - nw tokens.  idx [B][Hkv][k + window] int32 (device): the
 * min(k, n) tokens with the largest sigma among t < n (ties to the lower
 * index) in ascending order, then n, n + 1, ..., len - 1, then -1 -- the
 * whole row is ascending, and qattn_correct takes it with k + window as its k.
 * window == 0 is topk_select.  Size ws with bkv_workspace_bytes(layout,
 * max_len, k + window).  k + window == 0 enqueues nothing.
 * Errors: BKV_E_ARG if k < 0, window < 0 or k + window overflows int32;
 * BKV_E_CAPACITY for a bad length; BKV_E_WORKSPACE if ws is too small.
 */
bkv_status topk_select_window(const bkv_layout* layout, const float* sigma,
                              const int32_t* len_host, int32_t k,
                              int32_t window, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * topk_select_blocks -- block-granular selection: per (b, kvh) block j holds
 * tokens [j*block, min(len, j*block + block)) and scores the largest sigma
 * among them; the min(n_blocks, ceil(len/block)) best blocks are chosen, ties
 * to the lower block (Jet-QSparse abstract: the dense scan's scores select
 * 128-token blocks per KV head for exact fp16 value aggregation).
 * idx [B][Hkv][n_blocks * block] int32 (device): the chosen blocks in
 * ascending order, chosen block r as its tokens at idx[r*block ..
 * r*block + block) (-1 past len), then -1; qattn_correct takes it with
 * n_blocks * block as its k.  Uses the block-key region and the arrival
 * counters of ws: size it with bkv_workspace_bytes(layout, max_len,
 * n_blocks * block).  n_blocks == 0 enqueues nothing.
 * Errors: BKV_E_ARG unless block is a power of two in [32, 1024],
 * n_blocks >= 0 and n_blocks * block fits int32; BKV_E_UNSUPPORTED if
 * ceil(capacity / block) > 8192; BKV_E_CAPACITY for a bad length;
 * BKV_E_WORKSPACE if ws is too small.
 */
bkv_status topk_select_blocks(const bkv_layout* layout, const float* sigma,
                              const int32_t* len_host, int32_t n_blocks,
                              int32_t block, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * qattn_correct_blocks -- qattn_correct for the rows topk_select_blocks wrote
 * (same arguments as that call: n_blocks, block, and the same lengths), read
 * as whole blocks: the selected tokens' exact logits and fp16 values stream as
 * contiguous tiles of shadow rows (Jet-QSparse abstract: the chosen 128-token
 * blocks feed dense fp16 value aggregation with fp32 accumulation through
 * contiguous tile loads), logits on MFMA, the value sums in fp32, and their
 * approximate terms are recomputed by the scan's code over the same blocks.
 * out [B][Hq][D] fp32 as qattn_correct on these rows with n_blocks * block as
 * its k.  Needs qattn_decode_approx (or qattn_decode_select) of the same step
 * before it on ws, like qattn_correct.  Rows not written by
 * topk_select_blocks with these arguments give undefined results (every
 * access stays inside the cache).  The approximate terms run on a second
 * stream of the library's (one per device, default priority, made on the
 * first call and kept until the process ends), forked from and joined back
 * into `stream` with events; everything after the call on `stream` sees both
 * parts.
 * Errors: as topk_select_blocks's BKV_E_ARG; BKV_E_NULL, BKV_E_CAPACITY and
 * BKV_E_WORKSPACE (bkv_workspace_bytes(layout, max_len, n_blocks * block)) as
 * qattn_correct.
 */
bkv_status qattn_correct_blocks(const bkv_layout* layout, const bkv_cache* cache,
                                const uint16_t* q, const int32_t* len_host,
                                const int32_t* idx, int32_t n_blocks, int32_t block,
                                void* ws, size_t ws_bytes, float* out, void* stream);

/*
 * qattn_correct -- merge the splits written by qattn_decode_approx and apply
 * the exact correction (JetFire README, introduction: the approximate
 * attention over the low-bit cache is corrected for the top-k tokens with
 * their high-precision keys and values; standard softmax attention as in the
 * TailorKV review's Eq. 3): for the selected tokens S (idx, as written by
 * topk_select; negative entries are skipped) the approximate logit and value
 * are replaced by the exact ones from the shadow rows,
 *   lambda_t = (1/sqrt(D)) q . K_t,  nu_t = V_t        (t in S)
 *   lambda_t = s_hat[t],             nu_t = V_hat_t     (t not in S)
 *   out[b][h] = sum_t e^{lambda_t - m} nu_t / sum_t e^{lambda_t - m}  (fp32).
 * k == 0 gives the approximate output; idx may then be NULL.  A sequence with
 * len 0 gives zeros.  Entries outside [0, len) are skipped.  ws must hold the
 * split states written by qattn_decode_approx for the same lengths; the call
 * writes its chunk states into ws.
 * Errors: BKV_E_ARG if k < 0; BKV_E_WORKSPACE / BKV_E_CAPACITY as above.
 */
bkv_status qattn_correct(const bkv_layout* layout, const bkv_cache* cache,
                         const uint16_t* q, const int32_t* len_host,
                         const int32_t* idx, int32_t k, void* ws,
                         size_t ws_bytes, float* out, void* stream);

/*
 * qattn_score_select -- the selection scores and top-k rows of
 * qattn_decode_select (identical sigma and idx, same mode and workspace),
 * without the softmax state: the value codes are not read and no split state
 * is written.  The first pass of the exclusion path below.
 */
bkv_status qattn_score_select(const bkv_layout* layout, const bkv_cache* cache,
                              const uint16_t* q, const int32_t* len_host,
                              int32_t k, float* sigma, int32_t* idx, void* ws,
                              size_t ws_bytes, int32_t mode, void* stream);

/*
 * qattn_decode_unselected -- the approximate pass of qattn_decode_approx
 * restricted to the tokens that are NOT selected: per (b, kvh) the tokens
 * listed in the first min(k, len) entries of idx[b][kvh] (as topk_select
 * writes them; negative or out-of-range entries list nothing) are left out of
 * the split states it writes to ws; sigma is not written.  Together with
 * qattn_correct_unselected it computes the same output as qattn_correct, but
 * merges the exact terms of the selected tokens with a state that never
 * contained their approximate terms, instead of subtracting those: the
 * subtraction loses everything in fp32 when the selected tokens' approximate
 * weights dwarf the rest (as with 1- and 2-bit keys, whose approximate logits
 * can overshoot by tens of nats).  Costs a second pass over the packed cache.
 * Needs each scan range (split) at most 16384 tokens (BKV_E_UNSUPPORTED
 * otherwise); idx entries must be distinct.
 */
bkv_status qattn_decode_unselected(const bkv_layout* layout, const bkv_cache* cache,
                                   const uint16_t* q, const int32_t* len_host,
                                   const int32_t* idx, int32_t k, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * qattn_correct_unselected -- the output from the split states written by
 * qattn_decode_unselected (same idx, k, lengths and ws) and the exact terms of
 * the selected tokens: out = (sum over unselected of e^{s_hat} V_hat + sum over
 * selected of e^{s} V) / (the same sums of the weights), merged in log2
 * units without any subtraction.  Same arguments, workspace and errors as
 * qattn_correct.
 */
bkv_status qattn_correct_unselected(const bkv_layout* layout, const bkv_cache* cache,
                                    const uint16_t* q, const int32_t* len_host,
                                    const int32_t* idx, int32_t k, void* ws,
                                    size_t ws_bytes, float* out, void* stream);

/*
 * qattn_correct_hybrid -- qattn_correct with the exact half computed
 * elsewhere (JetFire README, introduction: "Approximate-then-Correct
 * Attention on Hybrid Memory" -- the high-precision copy lives in host memory
 * and the correction of the top-k tokens is computed from it there).
 * exact_state [B][Hq][2 + head_dim] fp32 (device): per (b, query head) the
 * exact softmax state of the selected tokens {m, l, a[0..D)} as
 * qattn_exact_host writes it (m in log2 units, -inf when no token is
 * selected).  The GPU computes only the selected tokens' approximate terms
 * (from the packed cache; the shadow is not read) and merges as
 * qattn_correct does.  Same workspace, idx and output contract as
 * qattn_correct; the cache's shadow pointers are not used.
 * Errors: as qattn_correct; BKV_E_NULL if exact_state is NULL.
 */
bkv_status qattn_correct_hybrid(const bkv_layout* layout, const bkv_cache* cache,
                                const uint16_t* q, const int32_t* len_host,
                                const int32_t* idx, int32_t k,
                                const float* exact_state, void* ws,
                                size_t ws_bytes, float* out, void* stream);

/*
 * qattn_hybrid_layers -- the hybrid step (qattn_decode_step, qattn_exact_host,
 * qattn_correct_hybrid; JetFire README, introduction: the correction of the
 * top-k tokens from the high-precision copy in host memory) over n_layers
 * layers, scheduled on the calling thread so that the host's exact passes
 * overlap GPU work.  The batch is split into `micro` micro-batches of
 * batch / micro consecutive rows (a layer's query depends on the previous
 * layer's output, so overlap comes from the other micro-batches): while the
 * host computes micro-batch m's states of layer i, the GPU runs the other
 * micro-batches' queued scans and merges.  Layer i appends (k_new[i],
 * v_new[i], [B][Hkv][D] fp16, device) at pos_host[b] and attends over
 * pos_host[b] + 1 tokens of caches[i] with q[i] ([B][Hq][D] fp16, device);
 * its output goes to out[i] ([B][Hq][D] fp32, device).  caches[i] must keep
 * its shadow rows in pinned host memory (bkv_cache).  slots[m]: micro-batch
 * m's buffers (layout with batch / micro rows): sigma, idx, a workspace of
 * bkv_workspace_bytes(that layout, max length, k) zero-filled once, state_dev
 * [B/micro][Hq][2 + D] fp32 (device), and pinned host idx_host, q_host,
 * state_host of the matching sizes.  The one call of the library that waits:
 * for each micro-batch's event (never for the whole stream); it creates and
 * destroys `micro` events.  Returns once every host pass is done and the
 * last merges are enqueued on `stream`.
 * Errors: BKV_E_NULL, BKV_E_ARG (n_layers, k, n_threads < 0, micro < 1 or
 * not dividing the batch), BKV_E_WORKSPACE, BKV_E_CAPACITY (a position
 * outside [0, capacity)) before anything is enqueued; later failures of
 * the calls it makes are returned as they come (work already enqueued
 * stays enqueued).
 */
typedef struct {
  float* sigma;        /* device [B/micro][Hkv][capacity]                   */
  int32_t* idx;        /* device [B/micro][Hkv][k]                          */
  void* ws;            /* device workspace                                  */
  size_t ws_bytes;
  float* state_dev;    /* device [B/micro][Hq][2 + D]                       */
  int32_t* idx_host;   /* pinned host [B/micro][Hkv][k]                     */
  uint16_t* q_host;    /* pinned host [B/micro][Hq][D]                      */
  float* state_host;   /* pinned host [B/micro][Hq][2 + D]                  */
} bkv_hybrid_slot;

bkv_status qattn_hybrid_layers(const bkv_layout* layout, int32_t n_layers,
                               const bkv_cache* caches, const uint16_t* const* q,
                               const uint16_t* const* k_new, const uint16_t* const* v_new,
                               const int32_t* pos_host, int32_t k, int32_t micro,
                               const bkv_hybrid_slot* slots, float* const* out,
                               int32_t n_threads, void* stream);

/*
 * qattn_exact_host -- HOST computation (runs on the calling thread and
 * n_threads OpenMP threads, 0 = the OpenMP default; returns when done) of the
 * exact state of the selected tokens for every (b, query head):
 *   lambda_t = log2(e)/sqrt(D) * q_h . K_t for t in S (the first min(k, len)
 *   entries of idx[b][kvh] that lie in [0, len)),
 *   state[b][h] = {m = max lambda, l = sum 2^(lambda - m),
 *                  a = sum 2^(lambda - m) V_t}     (m = -inf, l = a = 0 if S is empty)
 * in fp32.  All pointers are HOST pointers: k_shadow_host/v_shadow_host the
 * fp16 shadow rows in the cache's layout [B][Hkv][capacity][D] (e.g. the
 * pinned host shadow of a cache made for it, once the step's append has
 * completed), q_host [B][Hq][D] fp16, idx_host [B][Hkv][k], state_host
 * [B][Hq][2 + D] fp32.  Touches no GPU.
 * Errors: BKV_E_ARG if k < 0 or n_threads < 0; BKV_E_NULL; BKV_E_CAPACITY;
 * layout errors as everywhere.
 */
bkv_status qattn_exact_host(const bkv_layout* layout, const uint16_t* k_shadow_host,
                            const uint16_t* v_shadow_host, const uint16_t* q_host,
                            const int32_t* len_host, const int32_t* idx_host,
                            int32_t k, float* state_host, int32_t n_threads);

/*
 * qattn_decode_fused -- one whole decode step in ONE launch (JetFire README,
 * introduction: approximate attention over the low-bit cache, top-k
 * selection per KV head -- Jet-QSparse abstract: the budget is per KV head --
 * and exact correction of the selected tokens): optionally the append of one
 * token per sequence at len_host[b] - 1 (k_new, v_new [B][Hkv][D] fp16,
 * device, as qattn_decode_step; both NULL for no append), the approximate
 * scan, the per-(b, kvh) top-min(k, len) selection by sigma (ties to the
 * lower index) and the corrected output.  Results: sigma as
 * qattn_decode_approx, idx [B][Hkv][k] as topk_select (the same set and
 * order), out [B][Hq][D] fp32 as qattn_correct on that set (k == 0: the
 * approximate output; k >= len: exact attention).  The scan's workgroups of
 * a (b, kvh) pair meet at barriers inside the launch, so the grid must be
 * resident on the device at once; the call checks that and the shape.
 * Layouts: the fp16 query (query_bits 0) with affine keys of 3 or 4 bits, or
 * with MXFP4 keys (key_format 1 and 2, whose scores and correction follow
 * qattn_decode_approx and qattn_correct for that format).
 * Workspace: bkv_workspace_bytes(layout, max_len, k), zero-filled once
 * (the call keeps its counters and histograms at zero between calls).
 * Errors: BKV_E_UNSUPPORTED when the fused step cannot run this call (query
 * bits 8, k_bits < 3, MXFP4 keys of other than 4 bits, more than 256 (b, kvh)
 * pairs, more than 64 scan ranges per pair, ranges over 16384 tokens, ranges
 * per pair times k over 8192, or a grid larger than the device holds at once
 * -- nothing is
 * enqueued; bkv_fused_supported says which shapes qualify); BKV_E_NULL if
 * only one of k_new, v_new is NULL; otherwise as qattn_decode_step and
 * qattn_correct.
 */
bkv_status qattn_decode_fused(const bkv_layout* layout, const bkv_cache* cache,
                              const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* q, const int32_t* len_host, int32_t k,
                              float* sigma, int32_t* idx, float* out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * qattn_decode_fused_noalloc -- qattn_decode_fused without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a 64 MiB array inside the library, one per device, held from
 * the library's load until the process ends; the call allocates and frees
 * nothing.  Each call first clears the array's counters with a small kernel
 * on `stream` (no memset), then runs the same kernel as qattn_decode_fused;
 * results are the same.  Every call on a device shares that device's array:
 * calls that may overlap on one device (other streams, other threads) race
 * and must be serialised by the caller.
 * Errors: BKV_E_WORKSPACE if this step needs more than 64 MiB of workspace
 * (bkv_workspace_bytes with the call's max length and k; the 32K and 128K
 * headline shapes need about 12 and 46 MiB); otherwise as qattn_decode_fused.
 */
bkv_status qattn_decode_fused_noalloc(const bkv_layout* layout, const bkv_cache* cache,
                                      const uint16_t* k_new, const uint16_t* v_new,
                                      const uint16_t* q, const int32_t* len_host, int32_t k,
                                      float* sigma, int32_t* idx, float* out, void* stream);

/* Host only: *supported = 1 if the shape of a qattn_decode_fused call with
 * this layout, longest length max_len and k qualifies (the call can still
 * return BKV_E_UNSUPPORTED when the device cannot hold its grid at once). */
bkv_status bkv_fused_supported(const bkv_layout* layout, int32_t max_len, int32_t k,
                               int32_t* supported);

/* Static text for a status code. */
const char* bkv_status_string(bkv_status status);

#ifdef __cplusplus
}
#endif
#endif /* BITKV_H */
