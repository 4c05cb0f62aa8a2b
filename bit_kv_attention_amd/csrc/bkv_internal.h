// bkv_internal.h -- device helpers and kernel launchers of libbitkv.so (gfx950).
// Library-internal; the public surface is include/bitkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitkv.h"

namespace bkv {

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kGroups = kHeadDim / kGroup;  // 4
constexpr int kTile = 32;                   // tokens per V tile and per scan step
constexpr int kMaxBatch = 256;

// Per-sequence lengths / positions travel by value in the kernel arguments.
struct SeqArg {
  int32_t v[kMaxBatch];
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Byte sizes per unit (b, kvh).
__host__ __device__ inline size_t k_row_bytes(int kbits) { return (size_t)kHeadDim * kbits / 8; }
__host__ __device__ inline size_t k_unit_bytes(int kbits, int cap) { return (size_t)cap * k_row_bytes(kbits); }
__host__ __device__ inline size_t v_tile_bytes(int vbits) { return (size_t)kTile * kHeadDim * vbits / 8; }
__host__ __device__ inline size_t v_unit_bytes(int vbits, int cap) { return (size_t)(cap / kTile) * v_tile_bytes(vbits); }

// Order-preserving map of a float onto uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal values compare equal.
__device__ inline uint32_t float_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Split-L partial states inside the workspace.
struct Partials {
  float* m;    // [B][Hq][nsplit]  running max, log2 units
  float* l;    // [B][Hq][nsplit]  softmax denominator
  float* acc;  // [B][Hq][nsplit][D] unnormalised sum of p * V_hat
};

// Tokens per split for a step whose longest sequence has max_len tokens:
// a multiple of 4 waves * 32 tokens, sized for about 1024 workgroups.
int split_tokens(int units, int max_len);
int num_splits(int units, int max_len);
Partials partials_in(void* ws, int B, int Hq, int nsplit);
size_t partials_bytes(int B, int Hq, int nsplit);

// Launchers (return hipGetLastError of their launches).
hipError_t launch_pack_append(const bkv_layout& L, const bkv_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, int n_new, const SeqArg& pos, hipStream_t s);
hipError_t launch_decode_approx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                const SeqArg& len, int max_len, float* sigma, const Partials& p,
                                int nsplit, int chunk, hipStream_t s);
hipError_t launch_topk(const bkv_layout& L, const float* sigma, const SeqArg& len, int k,
                       int32_t* idx, hipStream_t s);
hipError_t launch_correct(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                          const SeqArg& len, const int32_t* idx, int k, const Partials& p,
                          int nsplit, float* out, hipStream_t s);

}  // namespace bkv
