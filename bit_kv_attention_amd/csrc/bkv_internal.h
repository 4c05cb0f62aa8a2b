// bkv_internal.h -- device helpers and kernel launchers of libbitkv.so (gfx950).
// Library-internal; the public surface is include/bitkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitkv.h"

namespace bkv {

constexpr int kHeadDim = 128;
// The kernels work on 32-channel quarters of a row (one MFMA K-step each).
// A quantisation group is one quarter (group 32) or two (group 64); the meta
// planes are per group, and quarter g reads group g >> mshift (mshift =
// log2(group / 32)).
constexpr int kGroup = 32;
constexpr int kGroups = kHeadDim / kGroup;  // 4 quarters
__host__ __device__ inline int meta_planes(int mshift) { return kGroups >> mshift; }
constexpr int kTile = 32;                   // tokens per V tile and per scan step
constexpr int kMaxBatch = 256;
constexpr int kScanWaves = 8;               // waves per workgroup of the approximate scan
constexpr int kScanWorkgroups = 256;        // target grid of the approximate scan

// Per-sequence lengths / positions travel by value in the kernel arguments.
struct SeqArg {
  int32_t v[kMaxBatch];
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---- packed layouts --------------------------------------------------------
// Keys: blocks of kKBlock tokens.  Channel c = 32g + 8e + j (group g, eighth
// e, offset j).  A block is 64 chunks in the order (e, token mod 16); chunk
// (e, r) holds the 32 codes of channels 32g + 8e + j of token r in the order
// (g, j), KB bits each (4*KB bytes).  So the 16 tokens x 4 eighths of a block
// are exactly the 64 lanes' A operands of a 16x16x32 MFMA tile, in lane order.
// Values: tiles of kTile tokens.  Token r of the tile is in quarter
// q = (r mod 16)/4 at slot j = 4(r/16) + r mod 4; channel c belongs to lane
// l = 16q + c mod 16 as its column n = c/16.  A dword holds 4/VB columns of
// one lane: column n in dword d = n/(4/VB) at sub-position s = n mod (4/VB),
// slot j at bit 16(j/4) + 4*VB*s + VB(j mod 4) -- so a right shift by 8s
// leaves the column in the layout the P.V MFMA unpack expects.  Dword d of
// lane l is dword 256(d/4) + 4l + d mod 4 of the tile (16-byte pieces,
// piece-major: each piece is one coalesced 1 KB load of a wave).
constexpr int kKBlock = 16;

__host__ __device__ inline size_t k_chunk_bytes(int kbits) { return (size_t)4 * kbits; }
__host__ __device__ inline size_t k_block_bytes(int kbits) { return (size_t)kKBlock * kHeadDim * kbits / 8; }
__host__ __device__ inline size_t k_unit_bytes(int kbits, int cap) { return (size_t)(cap / kKBlock) * k_block_bytes(kbits); }
__host__ __device__ inline size_t v_tile_bytes(int vbits) { return (size_t)kTile * kHeadDim * vbits / 8; }
__host__ __device__ inline size_t v_unit_bytes(int vbits, int cap) { return (size_t)(cap / kTile) * v_tile_bytes(vbits); }

// Byte offset, inside a unit's key codes, of the chunk (eighth e) of token t.
__host__ __device__ inline size_t k_chunk_offset(int kbits, int t, int e) {
  return (size_t)(t / kKBlock) * k_block_bytes(kbits) + (size_t)(e * kKBlock + t % kKBlock) * k_chunk_bytes(kbits);
}
// Key format 2 (MXFP4 keys scored against an MXFP4 query): a block of 16
// tokens is 64 chunks of 16 bytes; chunk 16g + (t mod 16) holds the 32 codes
// of channels 32g .. 32g+31 of token t, channel 32g + j in nibble j (low
// nibble first).  Lane l of a wave reading a block's 1 KB (16 bytes a lane)
// then holds the A operand (row = token l mod 16, K = 32(l/16) .. +31) of a
// 16x16x128 FP4 MFMA.  The scales are E8M0 bytes (2^(byte - 127)), one per
// (token, 32-channel block): word t of the unit's [capacity] uint32 plane
// holds block g's byte at bits 8g.
__host__ __device__ inline size_t k_chunk_offset_e8(int t, int g) {
  return (size_t)(t / kKBlock) * k_block_bytes(4) + (size_t)(16 * g + t % kKBlock) * 16;
}

// Dword index inside a value tile, and bit inside that dword, of the code of
// (token r of the tile, channel c).
__host__ __device__ inline void v_code_pos(int vbits, int r, int c, int& dw, int& bit) {
  const int q = (r & 15) >> 2, j = 4 * (r >> 4) + (r & 3);
  const int l = 16 * q + (c & 15), n = c >> 4;
  const int cpd = 4 / vbits, d = n / cpd, sub = n % cpd;
  dw = 256 * (d >> 2) + 4 * l + (d & 3);
  bit = 16 * (j >> 2) + 4 * vbits * sub + vbits * (j & 3);
}

// Order-preserving map of a float onto uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal values compare equal.
__device__ inline uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- workspace ------------------------------------------------------------
// One buffer: the top-k arrival counters (zero-filled once by the caller,
// left at zero by every call), the split partial states of the scan, the
// states of the correction chunks and the top-k candidate slots.  The
// region sizes depend on the step's longest length and k, so every call of a
// step recomputes the same offsets from the same (lens, k).

// Split-L partial states of the approximate scan.
struct Partials {
  float* m;    // [B][Hq][nsplit]  running max, log2 units
  float* l;    // [B][Hq][nsplit]  softmax denominator
  float* acc;  // [B][Hq][nsplit][D] unnormalised sum of p * V_hat
};

constexpr int kCorrChunk = 32;  // selected tokens per correction workgroup
// The correction of long rows of whole blocks (qattn_correct_blocks): one
// record per kRowRec row entries, its exact part from the shadow rows
// (correct.hip) and its approximate part from the scan's rows mode.
constexpr int kRowRec = 512;
// Per (b, h, chunk): m_exact, l_exact, m_approx, l_approx, then the exact and
// the approximate value sums (D each), 16-byte aligned.
constexpr int kCsStride = 4 + 2 * kHeadDim;
constexpr int kStateFloats = 2 + kHeadDim;  // one exact state {m, l, a[0..D)}

// Top-k: slices of S tokens (kTopkSliceMax, halved down to kTopkSliceMin
// while fewer than kTopkGridMin slice workgroups would run) whose local top-k
// candidates, ceil(max_len/S)*k slots per unit, must fit the merge's
// kTopkMergeMax; otherwise S = 0 selects the single-workgroup kernel.
constexpr int kTopkSliceMax = 8192;
constexpr int kTopkSliceMin = 2048;
constexpr int kTopkGridMin = 128;
constexpr int kTopkMergeMax = 16384;
constexpr int kTopkBlocksMax = 8192;  // blocks per unit for block selection (ceil(capacity / block))
constexpr int kTopkBlockSpan = 8192;  // tokens per workgroup of the block maxima
// Top-k inside the approximate scan: a split's scores staged in LDS, and the
// unit's candidate slots (nsplit * k) merged in LDS.
constexpr int kSelStage = 16384;
constexpr int kSelSlots = 8192;
constexpr int kSelMinRange = 8192;  // automatic mode: shorter ranges take two launches
int topk_slice(int units, int max_len, int k);

// The fused step (qattn_decode_fused): scan, selection, correction and output
// in one launch.  Its selection histograms the selection scores into kFBins
// bins of the top kFBinBits bits of their order-preserving keys (sign,
// exponent and 4 mantissa bits) per split in LDS; each split lists its
// highest entries in the workspace (fused_tail.h).  At most kFMaxSplits
// splits per unit and kFMaxUnits units.
constexpr int kFBinBits = 13;
constexpr int kFBins = 1 << kFBinBits;
constexpr int kFMaxSplits = 64;
constexpr int kFMaxUnits = 256;
constexpr int kFPass = 64;  // selected tokens per correction pass of the fused tail

// Workspace pointers of the fused step (all zero for the other launches).
struct FusedArgs {
  float* out;      // [B][Hq][D] the corrected output
  uint32_t* ctr;   // [U][2] arrival counters (zero between calls)
  uint64_t* dlist; // [U][nsplit][split length] each split's listed composites
  uint32_t* dcnt;  // [U][nsplit] list sizes
  uint32_t* dsv;   // [U][nsplit] the lowest bin each split lists
  uint32_t* flag;  // bit 0: a unit barrier gave up waiting (never expected)
};

struct Workspace {
  Partials part;
  float* cs;  // [B][Hq][nchunk][kCsStride]
  uint64_t* tkc;  // [U][top-k candidate slots] (composite keys)
  uint32_t* bkeys;  // [U][bkstride] block-selection keys
  int bkstride;
  uint32_t* tkctr;  // [U] arrivals of the top-k slice workgroups (zero between calls)
  FusedArgs fused;  // (out left null; null regions when the units exceed kFMaxUnits)
  int nsplit;
  int nchunk;
  size_t bytes;  // total bytes this step needs
};

// Tokens per split of the scan for a step whose longest sequence has max_len
// tokens: a multiple of 4 waves * 32 tokens, sized for about kScanWorkgroups.
int split_tokens(int units, int max_len);
int num_splits(int units, int max_len);
// Offsets of the regions for a step (ws may be null to size only).  With
// bound = true the split and chunk counts are upper bounds valid for every
// step whose longest sequence is at most max_len.
Workspace workspace_layout(void* ws, const bkv_layout& L, int max_len, int k, bool bound);

// Launchers (return hipGetLastError of their launches).
hipError_t launch_pack_append(const bkv_layout& L, const bkv_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, int n_new, const SeqArg& pos, hipStream_t s);
// ksel > 0: the same launch also writes the top-ksel rows to idx (its split
// length chunk <= kSelStage and nsplit * ksel <= kSelSlots).  skip: the
// split states leave out the tokens of the rows of idx (ksel entries per
// unit; chunk <= kSelStage); sigma is not written.  sigonly: only sigma (and
// with ksel > 0 the rows); no split states.  k_new/v_new (non-null, with
// neither skip nor sigonly): first append one token per sequence at len - 1.
hipError_t launch_decode_approx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                const SeqArg& len, float* sigma, const Workspace& w, int chunk,
                                int32_t* idx, int ksel, bool skip, bool sigonly, const uint16_t* k_new,
                                const uint16_t* v_new, hipStream_t s);
// The fused step: (append,) scan, top-ksel and correction into out, one
// launch whose workgroups of a unit meet at barriers.  hipErrorNotSupported
// when the layout has no fused kernel or the grid does not fit the device at
// once (nothing launched).
// Whether launch_decode_fused can run this layout and grid on the current
// device (the same test it makes before launching).
bool decode_fused_fits(const bkv_layout& L, const Workspace& w, bool append);
hipError_t launch_decode_fused(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                               float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel,
                               const uint16_t* k_new, const uint16_t* v_new, float* out, hipStream_t s);
// (the MXFP4 key formats' builds of the same: 1 fp16 query, 2 MXFP4 query)
bool decode_fused_fits_mx(const bkv_layout& L, const Workspace& w, bool append);
bool decode_fused_fits_fp4(const bkv_layout& L, const Workspace& w, bool append);
hipError_t launch_decode_fused_mx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                                  float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel,
                                  const uint16_t* k_new, const uint16_t* v_new, float* out, hipStream_t s);
hipError_t launch_decode_fused_fp4(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                                   float* sigma, const Workspace& w, int chunk, int32_t* idx, int ksel,
                                   const uint16_t* k_new, const uint16_t* v_new, float* out, hipStream_t s);
// The same with the INT8 query (layouts with query_bits = 8) and with MXFP4
// keys (key_format = 1); launch_decode_approx forwards those layouts here.
hipError_t launch_decode_approx_q8(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                   const SeqArg& len, float* sigma, const Workspace& w, int chunk,
                                   int32_t* idx, int ksel, bool skip, bool sigonly, const uint16_t* k_new,
                                   const uint16_t* v_new, hipStream_t s);
hipError_t launch_decode_approx_mx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                   const SeqArg& len, float* sigma, const Workspace& w, int chunk,
                                   int32_t* idx, int ksel, bool skip, bool sigonly, const uint16_t* k_new,
                                   const uint16_t* v_new, hipStream_t s);
// Key format 2: the scores on the scaled FP4 MFMA (decode_approx.hip built
// with BKV_KEY_FP4=1).
hipError_t launch_decode_approx_fp4(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                    const SeqArg& len, float* sigma, const Workspace& w, int chunk,
                                    int32_t* idx, int ksel, bool skip, bool sigonly, const uint16_t* k_new,
                                    const uint16_t* v_new, hipStream_t s);
// The approximate parts of the correction records of long block rows (row
// entries per unit; nrec records of kRowRec entries), one per build.
hipError_t launch_rows_approx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                              const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s);
hipError_t launch_rows_approx_q8(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                                 const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s);
hipError_t launch_rows_approx_mx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                                 const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s);
hipError_t launch_rows_approx_fp4(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                                  const Workspace& w, const int32_t* idx, int row, int nrec, hipStream_t s);
// qattn_correct on rows of whole blocks: the records' exact parts, their
// approximate parts (launch_rows_approx) and the merge into out.
hipError_t launch_correct_rows(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                               int max_len, const int32_t* idx, int row, const Workspace& w, float* out,
                               hipStream_t s);
// Rows of nb << lgb entries per unit: the nb best blocks of 1 << lgb tokens.
// bkeys: kstride block keys per unit; counter: one arrival counter per unit.
hipError_t launch_topk_blocks(const bkv_layout& L, const float* sigma, const SeqArg& len, int max_len, int nb,
                              int lgb, int32_t* idx, uint32_t* bkeys, int kstride, uint32_t* counter, hipStream_t s);
// Rows of k + W entries per unit (W: the recent window, 0 for none).
hipError_t launch_topk(const bkv_layout& L, const float* sigma, const SeqArg& len, int max_len, int k, int W,
                       int32_t* idx, uint64_t* cand, uint32_t* counter, hipStream_t s);
// hx: exact states from elsewhere ([B][Hq][kStateFloats]), or null.  rest:
// the split states already leave the selected tokens out (no subtraction).
hipError_t launch_correct(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                          const SeqArg& len, const int32_t* idx, int k, const Workspace& w,
                          const float* hx, bool rest, float* out, hipStream_t s);

}  // namespace bkv
