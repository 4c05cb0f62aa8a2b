// bitkv_api.hip -- the C ABI of libbitkv.so (declared in include/bitkv.h):
// host-side argument validation, workspace sizing and kernel launches.
// Nothing here allocates, frees or synchronises.
#include <math.h>
#include <string.h>

#include <mutex>

#include "bkv_internal.h"

namespace bkv {

// ---- the library-held workspace of qattn_decode_fused_noalloc -----------------
// One array per device, held from the library's load until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): it uses the address hipGetSymbolAddress
// returned on that device, kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Zero n words (a kernel, not a memset: callers may capture the launch into
// a graph).
__global__ void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int split_tokens(int units, int max_len) {
  // Work per workgroup: a multiple of kScanWaves waves x 32 tokens, sized so
  // the grid has about kScanWorkgroups workgroups when the context allows
  // (long runs per wave amortise the per-workgroup setup and merge).
  constexpr int q = kScanWaves * kTile;
  const long long total = (long long)units * (max_len > 0 ? max_len : 1);
  long long per = (total + kScanWorkgroups - 1) / kScanWorkgroups;
  per = ((per + q - 1) / q) * q;
  if (per < q) per = q;
  return (int)per;
}

int num_splits(int units, int max_len) {
  const int chunk = split_tokens(units, max_len);
  const int ns = (max_len + chunk - 1) / chunk;
  return ns > 0 ? ns : 1;
}

// An upper bound of num_splits(units, m) over every m <= max_len (the split
// count is not monotone in m): chunk >= q = kScanWaves*32 gives ceil(m/q),
// and chunk >= units*m/kScanWorkgroups gives ceil(kScanWorkgroups/units).
static int max_splits(int units, int max_len) {
  constexpr int q = kScanWaves * kTile;
  const int a = (max_len + q - 1) / q;
  const int b = (kScanWorkgroups + units - 1) / units;
  const int m = a < b ? a : b;
  return m > 0 ? m : 1;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int topk_slice(int units, int max_len, int k) {
  if (k <= 0) return 0;
  auto slots_for = [&](int S) { return (long long)((max_len + S - 1) / S) * k; };
  if (slots_for(kTopkSliceMax) > kTopkMergeMax) return 0;
  // halve the slices while the grid would leave compute units idle
  int S = kTopkSliceMax;
  while (S > kTopkSliceMin && (long long)units * ((max_len + S - 1) / S) < kTopkGridMin &&
         slots_for(S / 2) <= kTopkMergeMax)
    S /= 2;
  return S;
}

// Candidate slots per unit: ceil(max_len/S)*k <= ceil(max_len/kTopkSliceMin)*k,
// at most kTopkMergeMax when the two-kernel path runs -- a bound for every
// shorter step too (the region is sized even when this max_len itself takes
// the single-workgroup kernel).
static size_t topk_slots(int max_len, int k) {
  if (k <= 0) return 0;
  const long long a = (long long)((max_len + kTopkSliceMin - 1) / kTopkSliceMin) * k;
  return (size_t)(a < kTopkMergeMax ? a : kTopkMergeMax);
}

Workspace workspace_layout(void* ws, const bkv_layout& L, int max_len, int k, bool bound) {
  const int units = L.batch * L.n_kv_heads;
  Workspace w;
  w.nsplit = bound ? max_splits(units, max_len) : num_splits(units, max_len);
  const int kmax = k < max_len ? k : max_len;
  w.nchunk = kmax > 0 ? (kmax + kCorrChunk - 1) / kCorrChunk : 0;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off = align256(off + bytes);
    return p;
  };
  // Regions that must stay zero between calls come first, at offsets that
  // depend on the layout only (a later call with other lengths finds them in
  // place): the top-k arrival counters, the fused step's counters and its
  // flag word.
  w.tkctr = reinterpret_cast<uint32_t*>(take((size_t)units * 4));
  const bool fusable = units <= kFMaxUnits;
  w.fused = FusedArgs{};
  w.fused.ctr = reinterpret_cast<uint32_t*>(take((size_t)units * 2 * 4 + 4));
  if (w.fused.ctr) w.fused.flag = w.fused.ctr + (size_t)units * 2;
  const size_t recs = (size_t)L.batch * L.n_q_heads * w.nsplit;
  w.part.acc = reinterpret_cast<float*>(take(recs * kHeadDim * 4));
  w.part.m = reinterpret_cast<float*>(take(recs * 4));
  w.part.l = reinterpret_cast<float*>(take(recs * 4));
  w.cs = reinterpret_cast<float*>(take((size_t)L.batch * L.n_q_heads * w.nchunk * kCsStride * 4));
  // candidate slots: the top-k kernels', or the scan's own selection (nsplit
  // slots of k; used only when they fit kSelSlots, so that bounds them)
  size_t slots = topk_slots(max_len, k);
  if (k > 0) {
    const long long f = (long long)w.nsplit * k;
    const size_t fs = (size_t)(bound ? (f < kSelSlots ? f : kSelSlots) : (f <= kSelSlots ? f : 0));
    slots = fs > slots ? fs : slots;
  }
  w.tkc = reinterpret_cast<uint64_t*>(take((size_t)units * slots * 8));
  // block selection: one key per block of at least 32 tokens
  w.bkstride = (max_len + 31) / 32;
  w.bkeys = reinterpret_cast<uint32_t*>(take((size_t)units * w.bkstride * 4));
  if (fusable) {  // the fused step's per-split counts and threshold-bin lists
    w.fused.dcnt = reinterpret_cast<uint32_t*>(take((size_t)units * w.nsplit * 4));
    w.fused.dsv = reinterpret_cast<uint32_t*>(take((size_t)units * w.nsplit * 4));
    // one slot per token of each split: nsplit * split length < length + split
    // length (split length nondecreasing in the length), and the fused step
    // takes splits of at most kSelStage tokens
    const int chunk = split_tokens(units, max_len);
    const size_t per_unit = bound ? (size_t)max_len + (chunk < kSelStage ? chunk : kSelStage)
                                  : (chunk <= kSelStage ? (size_t)w.nsplit * chunk : 0);
    w.fused.dlist = reinterpret_cast<uint64_t*>(take((size_t)units * per_unit * 8));
  }
  w.bytes = off;
  return w;
}

}  // namespace bkv

using namespace bkv;

static bkv_status check_layout(const bkv_layout* L) {
  if (!L) return BKV_E_NULL;
  if (L->batch <= 0 || L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->head_dim <= 0 ||
      L->group <= 0 || L->capacity <= 0)
    return BKV_E_SHAPE;
  if (L->n_q_heads % L->n_kv_heads != 0) return BKV_E_SHAPE;
  if (L->head_dim % L->group != 0) return BKV_E_SHAPE;
  if (L->capacity % kTile != 0) return BKV_E_SHAPE;
  if (L->head_dim != kHeadDim || (L->group != kGroup && L->group != 2 * kGroup)) return BKV_E_UNSUPPORTED;
  if (L->k_bits < 1 || L->k_bits > 4) return BKV_E_UNSUPPORTED;
  if (L->v_bits != 2 && L->v_bits != 4) return BKV_E_UNSUPPORTED;
  const int G = L->n_q_heads / L->n_kv_heads;
  if (G != 4 && G != 8) return BKV_E_UNSUPPORTED;
  if (L->batch > kMaxBatch) return BKV_E_UNSUPPORTED;
  if (L->query_bits != 0 && L->query_bits != 8) return BKV_E_UNSUPPORTED;
  if (L->key_format < 0 || L->key_format > 2) return BKV_E_UNSUPPORTED;
  if (L->key_format != 0 && (L->k_bits != 4 || L->group != kGroup || L->query_bits != 0)) return BKV_E_UNSUPPORTED;
  return BKV_OK;
}

static bkv_status check_cache(const bkv_cache* c) {
  if (!c || !c->k_codes || !c->v_codes || !c->k_meta || !c->v_meta || !c->k_shadow || !c->v_shadow)
    return BKV_E_NULL;
  return BKV_OK;
}

static bkv_status read_lens(const bkv_layout* L, const int32_t* len_host, SeqArg* out, int* max_len) {
  if (!len_host) return BKV_E_NULL;
  int mx = 0;
  for (int b = 0; b < L->batch; ++b) {
    const int v = len_host[b];
    if (v < 0 || v > L->capacity) return BKV_E_CAPACITY;
    out->v[b] = v;
    mx = v > mx ? v : mx;
  }
  *max_len = mx;
  return BKV_OK;
}

extern "C" {

const char* bkv_status_string(bkv_status s) {
  switch (s) {
    case BKV_OK: return "ok";
    case BKV_E_NULL: return "a required pointer is NULL";
    case BKV_E_SHAPE: return "inconsistent shape";
    case BKV_E_UNSUPPORTED: return "unsupported configuration";
    case BKV_E_CAPACITY: return "position or length outside the cache capacity";
    case BKV_E_WORKSPACE: return "workspace too small";
    case BKV_E_HIP: return "HIP kernel launch failed";
    case BKV_E_ARG: return "invalid argument";
  }
  return "unknown status";
}

bkv_status bkv_cache_bytes(const bkv_layout* L, size_t* k_codes_bytes, size_t* v_codes_bytes,
                           size_t* meta_bytes_each, size_t* shadow_bytes_each) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!k_codes_bytes || !v_codes_bytes || !meta_bytes_each || !shadow_bytes_each) return BKV_E_NULL;
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  *k_codes_bytes = units * k_unit_bytes(L->k_bits, L->capacity);
  *v_codes_bytes = units * v_unit_bytes(L->v_bits, L->capacity);
  *meta_bytes_each = units * (size_t)(kHeadDim / L->group) * (size_t)L->capacity * sizeof(uint32_t);
  *shadow_bytes_each = units * (size_t)L->capacity * kHeadDim * sizeof(uint16_t);
  return BKV_OK;
}

bkv_status bkv_k_meta_bytes(const bkv_layout* L, size_t* bytes) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!bytes) return BKV_E_NULL;
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  *bytes = (L->key_format == 2) ? units * (size_t)L->capacity * sizeof(uint32_t)
                                : units * (size_t)(kHeadDim / L->group) * (size_t)L->capacity * sizeof(uint32_t);
  return BKV_OK;
}

bkv_status bkv_workspace_bytes(const bkv_layout* L, int32_t max_len, int32_t k, size_t* bytes) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!bytes) return BKV_E_NULL;
  if (max_len < 0 || max_len > L->capacity) return BKV_E_CAPACITY;
  if (k < 0) return BKV_E_ARG;
  *bytes = workspace_layout(nullptr, *L, max_len, k, true).bytes;
  return BKV_OK;
}

bkv_status kv_pack_append(const bkv_layout* L, const bkv_cache* c, const uint16_t* k_new,
                          const uint16_t* v_new, int32_t n_new, const int32_t* pos_host,
                          void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (!k_new || !v_new || !pos_host) return BKV_E_NULL;
  if (n_new < 0) return BKV_E_ARG;
  SeqArg pos;
  for (int b = 0; b < L->batch; ++b) {
    const int p = pos_host[b];
    if (p < 0 || (long long)p + n_new > L->capacity) return BKV_E_CAPACITY;
    pos.v[b] = p;
  }
  if (n_new == 0) return BKV_OK;
  return launch_pack_append(*L, *c, k_new, v_new, n_new, pos, (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status qattn_decode_approx(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                               const int32_t* len_host, float* sigma, void* ws, size_t ws_bytes,
                               void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (!q || !sigma || !ws) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, 0, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_decode_approx(*L, *c, q, len, sigma, w, split_tokens(units, max_len), nullptr, 0, false, false, nullptr, nullptr,
                              (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

// Whether qattn_decode_select selects inside the scan's launch: the layout
// must allow it (range <= kSelStage, nsplit * k <= kSelSlots); in the
// automatic mode the ranges must also be long (>= kSelMinRange), where
// rereading the scores in a launch of its own costs more than the selection
// in the scan's tail.
static bool select_in_scan(const Workspace& w, int chunk, int k, int mode) {
  if (k <= 0 || mode == 2 || chunk > kSelStage || (long long)w.nsplit * k > kSelSlots) return false;
  return mode == 1 || chunk >= kSelMinRange;
}

bkv_status bkv_select_in_scan(const bkv_layout* L, int32_t max_len, int32_t k, int32_t mode, int32_t* in_scan) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!in_scan) return BKV_E_NULL;
  if (max_len < 0 || max_len > L->capacity) return BKV_E_CAPACITY;
  if (k < 0 || mode < 0 || mode > 2) return BKV_E_ARG;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(nullptr, *L, max_len, k, false);
  *in_scan = select_in_scan(w, split_tokens(units, max_len), k, mode) ? 1 : 0;
  return BKV_OK;
}

bkv_status qattn_decode_select(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                               const int32_t* len_host, int32_t k, float* sigma, int32_t* idx, void* ws,
                               size_t ws_bytes, int32_t mode, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0 || mode < 0 || mode > 2) return BKV_E_ARG;
  if (!q || !sigma || !ws || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  const int chunk = split_tokens(units, max_len);
  const hipStream_t s = (hipStream_t)stream;
  if (select_in_scan(w, chunk, k, mode))
    return launch_decode_approx(*L, *c, q, len, sigma, w, chunk, idx, k, false, false, nullptr, nullptr, s) == hipSuccess ? BKV_OK
                                                                                                : BKV_E_HIP;
  if (launch_decode_approx(*L, *c, q, len, sigma, w, chunk, nullptr, 0, false, false, nullptr, nullptr, s) != hipSuccess) return BKV_E_HIP;
  if (k == 0) return BKV_OK;
  return launch_topk(*L, sigma, len, max_len, k, 0, idx, w.tkc, w.tkctr, s) == hipSuccess ? BKV_OK : BKV_E_HIP;
}

static bkv_status topk_rows(const bkv_layout* L, const float* sigma, const int32_t* len_host, int32_t k,
                            int32_t window, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (k < 0 || window < 0 || (long long)k + window > 0x7FFFFFFF) return BKV_E_ARG;
  const int row = k + window;
  if (!sigma || (!idx && row > 0) || (!ws && row > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  if (row == 0) return BKV_OK;
  const Workspace w = workspace_layout(ws, *L, max_len, row, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_topk(*L, sigma, len, max_len, k, window, idx, w.tkc, w.tkctr, (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status topk_select(const bkv_layout* L, const float* sigma, const int32_t* len_host, int32_t k,
                       int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return topk_rows(L, sigma, len_host, k, 0, idx, ws, ws_bytes, stream);
}

bkv_status topk_select_window(const bkv_layout* L, const float* sigma, const int32_t* len_host, int32_t k,
                              int32_t window, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return topk_rows(L, sigma, len_host, k, window, idx, ws, ws_bytes, stream);
}

bkv_status topk_select_blocks(const bkv_layout* L, const float* sigma, const int32_t* len_host,
                              int32_t n_blocks, int32_t block, int32_t* idx, void* ws, size_t ws_bytes,
                              void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (n_blocks < 0 || block < 32 || block > 1024 || (block & (block - 1)) != 0 ||
      (long long)n_blocks * block > 0x7FFFFFFF)
    return BKV_E_ARG;
  if ((L->capacity + block - 1) / block > kTopkBlocksMax) return BKV_E_UNSUPPORTED;
  if (!sigma || ((!idx || !ws) && n_blocks > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  if (n_blocks == 0) return BKV_OK;
  const Workspace w = workspace_layout(ws, *L, max_len, n_blocks * block, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  int lgb = 0;
  while ((1 << lgb) < block) ++lgb;
  return launch_topk_blocks(*L, sigma, len, max_len, n_blocks, lgb, idx, w.bkeys, w.bkstride, w.tkctr,
                            (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status qattn_correct(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                         const int32_t* len_host, const int32_t* idx, int32_t k, void* ws,
                         size_t ws_bytes, float* out, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0) return BKV_E_ARG;
  if (!q || !ws || !out || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_correct(*L, *c, q, len, idx, k, w, nullptr, false, out, (hipStream_t)stream) == hipSuccess ? BKV_OK
                                                                                                   : BKV_E_HIP;
}

bkv_status qattn_correct_blocks(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                                const int32_t* len_host, const int32_t* idx, int32_t n_blocks, int32_t block, void* ws,
                                size_t ws_bytes, float* out, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (n_blocks < 0 || block < 32 || block > 1024 || (block & (block - 1)) != 0 ||
      (long long)n_blocks * block > 0x7FFFFFFF)
    return BKV_E_ARG;
  const int row = n_blocks * block;
  if (!q || !ws || !out || (!idx && row > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const Workspace w = workspace_layout(ws, *L, max_len, row, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_correct_rows(*L, *c, q, len, max_len, idx, row, w, out, (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status qattn_decode_step(const bkv_layout* L, const bkv_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                             const uint16_t* q, const int32_t* len_host, int32_t k, float* sigma, int32_t* idx,
                             void* ws, size_t ws_bytes, int32_t mode, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0 || mode < 0 || mode > 2) return BKV_E_ARG;
  if (!k_new || !v_new || !q || !sigma || !ws || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  for (int b = 0; b < L->batch; ++b)
    if (len.v[b] < 1) return BKV_E_CAPACITY;  // the new token goes to len - 1
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  const int chunk = split_tokens(units, max_len);
  const hipStream_t s = (hipStream_t)stream;
  if (select_in_scan(w, chunk, k, mode))
    return launch_decode_approx(*L, *c, q, len, sigma, w, chunk, idx, k, false, false, k_new, v_new, s) ==
                   hipSuccess
               ? BKV_OK
               : BKV_E_HIP;
  if (launch_decode_approx(*L, *c, q, len, sigma, w, chunk, nullptr, 0, false, false, k_new, v_new, s) != hipSuccess)
    return BKV_E_HIP;
  if (k == 0) return BKV_OK;
  return launch_topk(*L, sigma, len, max_len, k, 0, idx, w.tkc, w.tkctr, s) == hipSuccess ? BKV_OK : BKV_E_HIP;
}

// Whether the fused step can run this call: an fp16 query with affine keys
// of 3 or 4 bits or MXFP4 keys (key formats 1 and 2), splits that fit the LDS
// stage, the per-split lists and the unit barriers' limits.
static bool fused_shape_ok(const bkv_layout* L, const Workspace& w, int chunk, int k) {
  const int units = L->batch * L->n_kv_heads;
  if (L->query_bits != 0 || L->k_bits < 3) return false;
  if (L->key_format != 0 && L->k_bits != 4) return false;
  if (units > kFMaxUnits || w.nsplit > kFMaxSplits || chunk > kSelStage) return false;
  return (long long)w.nsplit * k <= kSelSlots;
}

bkv_status bkv_fused_supported(const bkv_layout* L, int32_t max_len, int32_t k, int32_t* supported) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!supported) return BKV_E_NULL;
  if (max_len < 0 || max_len > L->capacity) return BKV_E_CAPACITY;
  if (k < 0) return BKV_E_ARG;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(nullptr, *L, max_len, k, false);
  *supported = fused_shape_ok(L, w, split_tokens(units, max_len), k) ? 1 : 0;
  return BKV_OK;
}

bkv_status qattn_decode_fused(const bkv_layout* L, const bkv_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* q, const int32_t* len_host, int32_t k, float* sigma, int32_t* idx,
                              float* out, void* ws, size_t ws_bytes, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0) return BKV_E_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return BKV_E_NULL;
  if (!q || !sigma || !out || !ws || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  if (k_new)
    for (int b = 0; b < L->batch; ++b)
      if (len.v[b] < 1) return BKV_E_CAPACITY;  // the new token goes to len - 1
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  const int chunk = split_tokens(units, max_len);
  if (!fused_shape_ok(L, w, chunk, k)) return BKV_E_UNSUPPORTED;
  const hipError_t e = launch_decode_fused(*L, *c, q, len, sigma, w, chunk, idx, k, k_new, v_new, out,
                                           (hipStream_t)stream);
  if (e == hipErrorNotSupported) return BKV_E_UNSUPPORTED;
  return e == hipSuccess ? BKV_OK : BKV_E_HIP;
}

bkv_status qattn_decode_fused_noalloc(const bkv_layout* L, const bkv_cache* c, const uint16_t* k_new,
                                      const uint16_t* v_new, const uint16_t* q, const int32_t* len_host, int32_t k,
                                      float* sigma, int32_t* idx, float* out, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0) return BKV_E_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return BKV_E_NULL;
  if (!q || !sigma || !out || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  if (k_new)
    for (int b = 0; b < L->batch; ++b)
      if (len.v[b] < 1) return BKV_E_CAPACITY;  // the new token goes to len - 1
  const int units = L->batch * L->n_kv_heads;
  const int chunk = split_tokens(units, max_len);
  const Workspace need = workspace_layout(nullptr, *L, max_len, k, false);
  if (need.bytes > kScratchBytes) return BKV_E_WORKSPACE;
  if (!fused_shape_ok(L, need, chunk, k)) return BKV_E_UNSUPPORTED;
  if (!decode_fused_fits(*L, need, k_new != nullptr)) return BKV_E_UNSUPPORTED;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return BKV_E_HIP;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  const hipStream_t s = (hipStream_t)stream;
  // the counters and the flag word, which lead the workspace, start at zero
  // (the array keeps whatever the last call on this device left)
  const size_t nz = (size_t)(reinterpret_cast<char*>(w.part.acc) - static_cast<char*>(ws)) / 4;
  (void)hipGetLastError();
  zero_words_kernel<<<dim3((unsigned)((nz + 255) / 256)), 256, 0, s>>>(static_cast<uint32_t*>(ws), nz);
  if (hipGetLastError() != hipSuccess) return BKV_E_HIP;
  const hipError_t e = launch_decode_fused(*L, *c, q, len, sigma, w, chunk, idx, k, k_new, v_new, out, s);
  if (e == hipErrorNotSupported) return BKV_E_UNSUPPORTED;
  return e == hipSuccess ? BKV_OK : BKV_E_HIP;
}

bkv_status qattn_score_select(const bkv_layout* L, const bkv_cache* c, const uint16_t* q, const int32_t* len_host,
                              int32_t k, float* sigma, int32_t* idx, void* ws, size_t ws_bytes, int32_t mode,
                              void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0 || mode < 0 || mode > 2) return BKV_E_ARG;
  if (!q || !sigma || !ws || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  const int chunk = split_tokens(units, max_len);
  const hipStream_t s = (hipStream_t)stream;
  if (select_in_scan(w, chunk, k, mode))
    return launch_decode_approx(*L, *c, q, len, sigma, w, chunk, idx, k, false, true, nullptr, nullptr, s) == hipSuccess ? BKV_OK
                                                                                               : BKV_E_HIP;
  if (launch_decode_approx(*L, *c, q, len, sigma, w, chunk, nullptr, 0, false, true, nullptr, nullptr, s) != hipSuccess) return BKV_E_HIP;
  if (k == 0) return BKV_OK;
  return launch_topk(*L, sigma, len, max_len, k, 0, idx, w.tkc, w.tkctr, s) == hipSuccess ? BKV_OK : BKV_E_HIP;
}

bkv_status qattn_decode_unselected(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                                   const int32_t* len_host, const int32_t* idx, int32_t k, void* ws,
                                   size_t ws_bytes, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0) return BKV_E_ARG;
  if (!q || !ws || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const int units = L->batch * L->n_kv_heads;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  const int chunk = split_tokens(units, max_len);
  if (chunk > kSelStage) return BKV_E_UNSUPPORTED;
  return launch_decode_approx(*L, *c, q, len, nullptr, w, chunk, const_cast<int32_t*>(idx), k, true, false, nullptr, nullptr,
                              (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status qattn_correct_unselected(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                                    const int32_t* len_host, const int32_t* idx, int32_t k, void* ws,
                                    size_t ws_bytes, float* out, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if ((st = check_cache(c)) != BKV_OK) return st;
  if (k < 0) return BKV_E_ARG;
  if (!q || !ws || !out || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_correct(*L, *c, q, len, idx, k, w, nullptr, true, out, (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

bkv_status qattn_correct_hybrid(const bkv_layout* L, const bkv_cache* c, const uint16_t* q,
                                const int32_t* len_host, const int32_t* idx, int32_t k, const float* exact_state,
                                void* ws, size_t ws_bytes, float* out, void* stream) {
  bkv_status st = check_layout(L);
  if (st != BKV_OK) return st;
  if (!c || !c->k_codes || !c->v_codes || !c->k_meta || !c->v_meta) return BKV_E_NULL;
  if (k < 0) return BKV_E_ARG;
  if (!q || !ws || !out || !exact_state || (!idx && k > 0)) return BKV_E_NULL;
  SeqArg len;
  int max_len = 0;
  if ((st = read_lens(L, len_host, &len, &max_len)) != BKV_OK) return st;
  const Workspace w = workspace_layout(ws, *L, max_len, k, false);
  if (ws_bytes < w.bytes) return BKV_E_WORKSPACE;
  return launch_correct(*L, *c, q, len, idx, k, w, exact_state, false, out, (hipStream_t)stream) == hipSuccess
             ? BKV_OK
             : BKV_E_HIP;
}

}  // extern "C"
