// pack.hip -- quantise and store appended tokens (the quantiser itself, and
// why it is bit-exact, is in quant_lane.h): the codes go into the packed
// layouts, (s, z) into the meta planes and the fp16 row verbatim into the
// shadow.
//
// One workgroup per (32-token tile, unit); 32 lanes per token (16 for K, 16
// for V, four per 32-channel quarter).  A lane's 8 key codes are exactly one
// quarter's share of one key chunk (4*KB bytes: its eighth of each of the 4
// quarters), so keys go straight to HBM.  Value dwords mix 8 tokens and are
// rebuilt from codes in LDS with a read-modify-write (slots of tokens outside
// the append keep their bits); their loads are issued before the quantiser
// runs.
#include "bkv_internal.h"
#include "quant_lane.h"

// The codec must match a plain IEEE evaluation operation for operation.
#pragma clang fp contract(off)

namespace bkv {
namespace {

// KF: the key format -- 0 affine codes (quantise_lane), 1 MXFP4 with fp16
// scales (quantise_lane_mx), 2 MXFP4 with E8M0 scales in the 32-channel chunk
// layout (quantise_lane_e8, one scale byte per token and quarter).
template <int KB, int VB, int KF = 0>
__global__ __launch_bounds__(256) void pack_append_kernel(
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, uint32_t* __restrict__ k_meta,
    uint32_t* __restrict__ v_meta, uint16_t* __restrict__ k_shadow, uint16_t* __restrict__ v_shadow,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int n_new, SeqArg pos,
    int Hkv, int cap, int mshift) {
  const int u = __builtin_amdgcn_workgroup_id_y();
  const int b = u / Hkv;
  const int p0 = pos.v[b];
  const int tile = p0 / kTile + (int)__builtin_amdgcn_workgroup_id_x();
  const int t0 = tile * kTile;
  const int t_lo = max(p0, t0);
  const int t_hi = min(p0 + n_new, t0 + kTile);
  if (t_lo >= t_hi) return;
  const int tid = __builtin_amdgcn_workitem_id_x();

  // value dwords this thread rebuilds: dword w of the tile is dword
  // d = 4(w/256) + w mod 4 of lane l = (w/4) mod 64, which holds the slots of
  // tokens 4q..4q+3 and 16+4q..16+4q+3 (q = l/16) for 4/VB columns
  constexpr int kWords = kHeadDim * VB / 256;  // per thread
  constexpr int kCpd = 4 / VB;
  uint32_t* vt = reinterpret_cast<uint32_t*>(v_codes + (size_t)u * v_unit_bytes(VB, cap) +
                                             (size_t)tile * v_tile_bytes(VB));
  uint32_t word[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) word[i] = vt[tid + 256 * i];

  __shared__ uint8_t s_vcode[kTile][kHeadDim];  // value codes [token][channel]
  const int sub = tid & 3, grp = (tid >> 2) & 3, kv = (tid >> 4) & 1;
  const int c0 = grp * kGroup + sub * 8;  // first channel of this lane
  const float qmax = (float)((1 << (kv ? VB : KB)) - 1);
  for (int r = (t_lo - t0) & ~7; r < t_hi - t0; r += 8) {
    const int t = t0 + r + (tid >> 5);
    if (t < t_lo || t >= t_hi) continue;
    const uint16_t* src = (kv ? v_new : k_new) + ((size_t)u * n_new + (t - p0)) * kHeadDim + c0;
    const uint4 w4 = *reinterpret_cast<const uint4*>(src);
    float x[8];
    halves8(w4, x);
    uint32_t code[8];
    const uint32_t meta = (KF == 1 && kv == 0)   ? quantise_lane_mx(x, code)
                          : (KF == 2 && kv == 0) ? quantise_lane_e8(x, code)
                                                 : quantise_lane(x, sub, grp, mshift, qmax, code);
    if (KF == 2 && kv == 0) {
      if (sub == 0) reinterpret_cast<uint8_t*>(k_meta)[((size_t)u * cap + t) * kGroups + grp] = (uint8_t)meta;
    } else if (sub == 0 && (grp & ((1 << mshift) - 1)) == 0) {
      (kv ? v_meta : k_meta)[((size_t)u * meta_planes(mshift) + (grp >> mshift)) * cap + t] = meta;
    }
    *reinterpret_cast<uint4*>((kv ? v_shadow : k_shadow) + ((size_t)u * cap + t) * kHeadDim + c0) = w4;
    if (kv == 0) {
      if constexpr (KF == 2)
        store_key_codes_e8(k_codes + (size_t)u * k_unit_bytes(KB, cap), t, sub, grp, code);
      else
        store_key_codes<KB>(k_codes + (size_t)u * k_unit_bytes(KB, cap), t, sub, grp, code);
    } else {
      uint2 cw;
      cw.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      cw.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
      *reinterpret_cast<uint2*>(&s_vcode[r + (tid >> 5)][c0]) = cw;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    const int w = tid + 256 * i;
    const int l = (w >> 2) & 63, d = 4 * (w >> 8) + (w & 3), qq = l >> 4;
    bool touched = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = (j < 4) ? (4 * qq + j) : (16 + 4 * qq + (j - 4));
      const int tt = t0 + rr;
      if (tt < t_lo || tt >= t_hi) continue;
      touched = true;
#pragma unroll
      for (int sb = 0; sb < kCpd; ++sb) {
        const int c = 16 * (d * kCpd + sb) + (l & 15);
        const int bit = 16 * (j >> 2) + 4 * VB * sb + VB * (j & 3);
        const uint32_t m = ((1u << VB) - 1) << bit;
        word[i] = (word[i] & ~m) | ((uint32_t)s_vcode[rr][c] << bit);
      }
    }
    if (touched) vt[w] = word[i];
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
  if (KB == 4 && L.key_format == 1)
    pack_append_kernel<KB, VB, 1><<<grid, 256, 0, s>>>(
        static_cast<uint8_t*>(c.k_codes), static_cast<uint8_t*>(c.v_codes), c.k_meta, c.v_meta,
        c.k_shadow, c.v_shadow, k_new, v_new, n_new, pos, L.n_kv_heads, L.capacity, 0);
  else if (KB == 4 && L.key_format == 2)
    pack_append_kernel<KB, VB, 2><<<grid, 256, 0, s>>>(
        static_cast<uint8_t*>(c.k_codes), static_cast<uint8_t*>(c.v_codes), c.k_meta, c.v_meta,
        c.k_shadow, c.v_shadow, k_new, v_new, n_new, pos, L.n_kv_heads, L.capacity, 0);
  else
    pack_append_kernel<KB, VB><<<grid, 256, 0, s>>>(
        static_cast<uint8_t*>(c.k_codes), static_cast<uint8_t*>(c.v_codes), c.k_meta, c.v_meta,
        c.k_shadow, c.v_shadow, k_new, v_new, n_new, pos, L.n_kv_heads, L.capacity, L.group == 64 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_append(const bkv_layout& L, const bkv_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, int n_new, const SeqArg& pos, hipStream_t s) {
  const bool v4 = L.v_bits == 4;
  switch (L.k_bits) {
    case 4: return v4 ? launch_kv<4, 4>(L, c, k_new, v_new, n_new, pos, s) : launch_kv<4, 2>(L, c, k_new, v_new, n_new, pos, s);
    case 3: return v4 ? launch_kv<3, 4>(L, c, k_new, v_new, n_new, pos, s) : launch_kv<3, 2>(L, c, k_new, v_new, n_new, pos, s);
    case 2: return v4 ? launch_kv<2, 4>(L, c, k_new, v_new, n_new, pos, s) : launch_kv<2, 2>(L, c, k_new, v_new, n_new, pos, s);
    default: return v4 ? launch_kv<1, 4>(L, c, k_new, v_new, n_new, pos, s) : launch_kv<1, 2>(L, c, k_new, v_new, n_new, pos, s);
  }
}

}  // namespace bkv
