// pack.hip -- quantise and store appended tokens.
//
// Per token, per K/V, per group of 32 channels (the asymmetric per-group
// quantiser of the HACK review on Pith, Eq. (4): zero point = group minimum,
// step = range / (2^b - 1); fp16 zero point and scale as in the TailorKV
// review's free-parameter list):
//   z = min x,  s = fp16((max - min) / (2^b - 1))   [fp32 subtract, IEEE divide]
//   code = clamp(rint((x - z) / s), 0, 2^b - 1)     [stored fp16 s and z; 0 if s == 0]
// then the codes go into the packed layouts, (s, z) into the meta planes and
// the fp16 row verbatim into the shadow.  Min/max run sequentially over the
// group in channel order (same tie behaviour for +-0 as a plain loop).
//
// One workgroup per (32-token tile, unit): thread (token r, K/V, group)
// quantises one group and leaves its codes in LDS; then one thread per key
// chunk (one token's codes of one eighth of every group) writes that chunk
// whole, and value words, which mix 8 tokens, are assembled with a
// read-modify-write of the tile's words (tokens outside the append keep
// their bits).
#include "bkv_internal.h"

// The codec must match a plain IEEE evaluation operation for operation.
#pragma clang fp contract(off)

namespace bkv {
namespace {

template <int KB, int VB>
__global__ __launch_bounds__(256) void pack_append_kernel(
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, uint32_t* __restrict__ k_meta,
    uint32_t* __restrict__ v_meta, uint16_t* __restrict__ k_shadow, uint16_t* __restrict__ v_shadow,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int n_new, SeqArg pos,
    int Hkv, int cap) {
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int p0 = pos.v[b];
  const int tile = p0 / kTile + blockIdx.x;
  const int t_lo = max(p0, tile * kTile);
  const int t_hi = min(p0 + n_new, tile * kTile + kTile);
  if (t_lo >= t_hi) return;

  __shared__ uint8_t s_code[2][kTile][kHeadDim];  // [K/V][token][channel]
  const int tid = threadIdx.x;
  const int r = tid >> 3;
  const int kv = (tid >> 2) & 1;
  const int grp = tid & 3;
  const int t = tile * kTile + r;
  if (t >= t_lo && t < t_hi) {
    const int bits = kv ? VB : KB;
    const uint16_t* src = (kv ? v_new : k_new) + ((size_t)u * n_new + (t - p0)) * kHeadDim + grp * kGroup;
    uint16_t x[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; i += 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[i + 2 * j] = (uint16_t)(ww[j] & 0xFFFFu);
        x[i + 2 * j + 1] = (uint16_t)(ww[j] >> 16);
      }
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float v = (float)__builtin_bit_cast(_Float16, x[i]);
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    const float qmax = (float)((1 << bits) - 1);
    const float s32 = (mx - mn) / qmax;
    const _Float16 s16 = (_Float16)s32;
    const _Float16 z16 = (_Float16)mn;
    const float s = (float)s16, z = (float)z16;
    uint8_t code[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      int cd = 0;
      if (s != 0.0f) {
        const float v = (float)__builtin_bit_cast(_Float16, x[i]);
        const float rr = __builtin_rintf((v - z) / s);
        cd = rr < 0.0f ? 0 : (rr > qmax ? (int)qmax : (int)rr);
      }
      code[i] = (uint8_t)cd;
    }
    const uint32_t meta = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
    (kv ? v_meta : k_meta)[((size_t)u * kGroups + grp) * cap + t] = meta;
    uint16_t* dst = (kv ? v_shadow : k_shadow) + ((size_t)u * cap + t) * kHeadDim + grp * kGroup;
#pragma unroll
    for (int i = 0; i < kGroup; i += 8)
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) s_code[kv][r][grp * kGroup + i] = code[i];
  }
  __syncthreads();
  // key chunks: chunk (eighth e, token r) of the 16-token block holds the
  // codes of channels 32g + 8e + j, packed in the order (g, j) at KB bits
  // each -- 4*KB bytes, written whole by one thread.
  if (tid < 4 * kTile) {
    const int rr = tid & (kTile - 1), e = tid >> 5;
    const int tt = tile * kTile + rr;
    if (tt >= t_lo && tt < t_hi) {
      uint32_t w[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) w[j] = 0;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const uint32_t cd = s_code[0][rr][32 * (m >> 3) + 8 * e + (m & 7)];
        const int bp = m * KB;
        w[bp >> 5] |= cd << (bp & 31);
        if ((bp & 31) + KB > 32) w[(bp >> 5) + 1] |= cd >> (32 - (bp & 31));
      }
      uint32_t* chunk = reinterpret_cast<uint32_t*>(
          k_codes + (size_t)u * k_unit_bytes(KB, cap) + (size_t)(tt / kKBlock) * k_block_bytes(KB) +
          (size_t)(e * kKBlock + (tt % kKBlock)) * k_chunk_bytes(KB));
#pragma unroll
      for (int j = 0; j < KB; ++j) chunk[j] = w[j];
    }
  }
  // value dwords: dword w of the tile belongs to lane l = (w/4) mod 64 as its
  // dword d = 4(w/256) + w mod 4, i.e. columns n = d*cpd + s (s < cpd) of
  // quarter l/16; only the slots of appended tokens are replaced
  constexpr int kCpd = 4 / VB;
  uint32_t* vt = reinterpret_cast<uint32_t*>(v_codes + (size_t)u * v_unit_bytes(VB, cap) +
                                             (size_t)tile * v_tile_bytes(VB));
  for (int w = tid; w < kHeadDim * VB; w += 256) {
    const int l = (w >> 2) & 63, d = 4 * (w >> 8) + (w & 3), qq = l >> 4;
    uint32_t word = vt[w];
#pragma unroll
    for (int sub = 0; sub < kCpd; ++sub) {
      const int c = 16 * (d * kCpd + sub) + (l & 15);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rr = (j < 4) ? (4 * qq + j) : (16 + 4 * qq + (j - 4));
        const int tt = tile * kTile + rr;
        if (tt >= t_lo && tt < t_hi) {
          const int bit = 16 * (j >> 2) + 4 * VB * sub + VB * (j & 3);
          const uint32_t m = ((1u << VB) - 1) << bit;
          word = (word & ~m) | ((uint32_t)s_code[1][rr][c] << bit);
        }
      }
    }
    vt[w] = word;
  }
}

template <int KB, int VB>
hipError_t launch_kv(const bkv_layout& L, const bkv_cache& c, const uint16_t* k_new,
                     const uint16_t* v_new, int n_new, const SeqArg& pos, hipStream_t s) {
  int tiles = 0;
  for (int b = 0; b < L.batch; ++b) {
    const int first = pos.v[b] / kTile;
    const int last = (pos.v[b] + n_new - 1) / kTile;
    tiles = tiles > (last - first + 1) ? tiles : (last - first + 1);
  }
  dim3 grid(tiles, L.batch * L.n_kv_heads);
  (void)hipGetLastError();  // report only this launch's status
  pack_append_kernel<KB, VB><<<grid, 256, 0, s>>>(
      static_cast<uint8_t*>(c.k_codes), static_cast<uint8_t*>(c.v_codes), c.k_meta, c.v_meta,
      c.k_shadow, c.v_shadow, k_new, v_new, n_new, pos, L.n_kv_heads, L.capacity);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_append(const bkv_layout& L, const bkv_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, int n_new, const SeqArg& pos, hipStream_t s) {
  if (L.k_bits == 4 && L.v_bits == 4) return launch_kv<4, 4>(L, c, k_new, v_new, n_new, pos, s);
  if (L.k_bits == 4 && L.v_bits == 2) return launch_kv<4, 2>(L, c, k_new, v_new, n_new, pos, s);
  if (L.k_bits == 3 && L.v_bits == 4) return launch_kv<3, 4>(L, c, k_new, v_new, n_new, pos, s);
  return launch_kv<3, 2>(L, c, k_new, v_new, n_new, pos, s);
}

}  // namespace bkv
