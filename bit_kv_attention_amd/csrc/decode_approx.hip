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
// Mapping onto gfx950 (one workgroup = 4 waves = one (b, kvh) unit and one
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
//  * Codes become fp16 integers with one AND-OR against 0x6400 (1024 + code)
//    and one packed fp16 subtract of 1024, both exact.
#include "bkv_internal.h"

namespace bkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// DPP helpers (row = 16 lanes).
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Two codes (one per 16-bit half, already masked) -> exact fp16 integers.
__device__ inline uint32_t codes_to_half2(uint32_t two_codes) {
  const uint32_t biased = two_codes | 0x64006400u;  // fp16 1024 + code in each half
  half2_t h = __builtin_bit_cast(half2_t, biased);
  h = h - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, h);
}

// y holds 4 codes of `BITS` bits in its low half and 4 in its high half; item
// pair r of the operand is (code r, code r+4).
template <int BITS>
__device__ inline half8 unpack8(uint32_t y) {
  constexpr uint32_t M = (BITS == 4) ? 0x000F000Fu : (BITS == 3) ? 0x00070007u : 0x00030003u;
  u32x4 r;
  r.x = codes_to_half2(y & M);
  r.y = codes_to_half2((y >> BITS) & M);
  r.z = codes_to_half2((y >> (2 * BITS)) & M);
  r.w = codes_to_half2((y >> (3 * BITS)) & M);
  return __builtin_bit_cast(half8, r);
}

__device__ inline float lo_half(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ inline float hi_half(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ inline uint32_t pack_half2(float lo, float hi) {
  half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

template <int KB, int VB, int G>
struct Step {
  static constexpr int NT = (G == 8) ? 2 : 1;
  static constexpr int KW = (KB == 4) ? 1 : 2;
  uint32_t kc[2][kGroups][KW];  // key code dwords: [token tile][group][dword]
  u32x4 km[2][NT];              // key meta, tokens 4kb..4kb+3 of token tile tt
  uint32_t vc[8];               // value word (channel 16*nt + n, quarter kb)
  u32x4 vm[NT][2];              // value meta: [N-tile][token tile]
};

template <int KB, int VB, int G>
__device__ inline void load_step(Step<KB, VB, G>& S, const uint8_t* __restrict__ kbase,
                                 const uint8_t* __restrict__ vbase, const uint32_t* __restrict__ kmeta,
                                 const uint32_t* __restrict__ vmeta, int cap, int t0, int n, int kb) {
  constexpr int NT = Step<KB, VB, G>::NT;
  constexpr int RB = kHeadDim * KB / 8;  // bytes per key row
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const uint32_t* row = reinterpret_cast<const uint32_t*>(kbase + (size_t)(t0 + 16 * tt + n) * RB);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if constexpr (KB == 4) {
        S.kc[tt][g][0] = row[4 * g + kb];
      } else {
        const int d0 = 3 * g + ((24 * kb) >> 5);
        const int d1 = min(d0 + 1, 3 * g + 2);
        S.kc[tt][g][0] = row[d0];
        S.kc[tt][g][1] = row[d1];
      }
    }
  }
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int gq = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      S.km[tt][T] = *reinterpret_cast<const u32x4*>(kmeta + (size_t)gq * cap + t0 + 16 * tt + 4 * kb);
      S.vm[T][tt] = *reinterpret_cast<const u32x4*>(vmeta + (size_t)gq * cap + t0 + 16 * tt + 4 * kb);
    }
  }
  const uint8_t* vt = vbase + (size_t)(t0 / kTile) * v_tile_bytes(VB);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int w = (16 * nt + n) * 4 + kb;
    if constexpr (VB == 4)
      S.vc[nt] = reinterpret_cast<const uint32_t*>(vt)[w];
    else
      S.vc[nt] = reinterpret_cast<const uint16_t*>(vt)[w];
  }
}

template <int KB, int VB, int G>
__global__ __launch_bounds__(256) void decode_approx_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const uint32_t* __restrict__ k_meta, const uint32_t* __restrict__ v_meta,
    const uint16_t* __restrict__ q, float* __restrict__ sigma, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ pacc, SeqArg lens, int Hq, int Hkv, int cap,
    int nsplit, int chunk) {
  constexpr int NT = Step<KB, VB, G>::NT;
  const int u = blockIdx.y;
  const int b = u / Hkv;
  const int kvh = u - b * Hkv;
  const int split = blockIdx.x;
  const int len = lens.v[b];
  const int t_begin = split * chunk;
  const int t_end = min(len, t_begin + chunk);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15;
  const int kb = lane >> 4;

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  const uint32_t* kmeta = k_meta + (size_t)u * kGroups * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * kGroups * cap;
  const uint16_t* qg = q + ((size_t)b * Hq + (size_t)kvh * G) * kHeadDim;

  // ---- query operands: column (g', h) of N-tile T --------------------------
  const int h = (G == 8) ? (n & 7) : (n & 3);
  half8 bq[kGroups];
  float qs[NT];
  {
    const uint16_t* qh = qg + (size_t)h * kHeadDim;
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const int gq = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
      float s = 0.f;
      for (int c = 0; c < kGroup; ++c) s += (float)__builtin_bit_cast(_Float16, qh[gq * kGroup + c]);
      qs[T] = s;
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int gq = (G == 8) ? (2 * (g >> 1) + (n >> 3)) : (n >> 2);
      half8 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint16_t a = qh[g * kGroup + 8 * kb + r];
        const uint16_t c = qh[g * kGroup + 8 * kb + 4 + r];
        v[2 * r] = (gq == g) ? __builtin_bit_cast(_Float16, a) : (_Float16)0.0f;
        v[2 * r + 1] = (gq == g) ? __builtin_bit_cast(_Float16, c) : (_Float16)0.0f;
      }
      bq[g] = v;
    }
  }

  const float sm = 1.0f / sqrtf((float)kHeadDim);
  const float sm2 = sm * kLog2e;

  // ---- running state --------------------------------------------------------
  float m_run = -INFINITY;
  float l_part = 0.f;
  float z_part[NT];
  floatx4 acc[8];
#pragma unroll
  for (int T = 0; T < NT; ++T) z_part[T] = 0.f;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = (floatx4){0.f, 0.f, 0.f, 0.f};

  Step<KB, VB, G> cur, nxt;
  int t0 = t_begin + kTile * wv;
  if (t0 < t_end) load_step<KB, VB, G>(cur, kbase, vbase, kmeta, vmeta, cap, t0, n, kb);

  for (; t0 < t_end; t0 += 4 * kTile) {
    const bool more = (t0 + 4 * kTile) < t_end;
    if (more) load_step<KB, VB, G>(nxt, kbase, vbase, kmeta, vmeta, cap, t0 + 4 * kTile, n, kb);

    // -- scores: D[T][tt] rows = tokens 4kb+i of token tile tt, column n ------
    floatx4 d[NT][2];
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) d[T][tt] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        uint32_t y;
        if constexpr (KB == 4) {
          y = cur.kc[tt][g][0];
        } else {
          const int shift = (24 * kb) & 31;
          const uint32_t x = __builtin_amdgcn_alignbit(cur.kc[tt][g][1], cur.kc[tt][g][0], shift);
          y = (x & 0xFFFFu) | ((x << 4) & 0xFFFF0000u);
        }
        const half8 a = unpack8<KB>(y);
        const int T = (G == 8) ? (g >> 1) : 0;
        d[T][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[g], d[T][tt], 0, 0, 0);
      }
    }

    // -- per-(token, group) scale and zero, reduce over groups ----------------
    float s2[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float part = 0.f;
#pragma unroll
        for (int T = 0; T < NT; ++T) {
          const uint32_t mw = cur.km[tt][T][i];
          part += d[T][tt][i] * lo_half(mw) + hi_half(mw) * qs[T];
        }
        if constexpr (G == 8) {
          part += dpp<kRowRor8>(part);
        } else {
          part += dpp<kRowRor4>(part);
          part += dpp<kRowRor8>(part);
        }
        const int t = t0 + 16 * tt + 4 * kb + i;
        const bool valid = t < len;
        // selection score: max over the query heads of the group
        float sg = part * sm;
        sg = fmaxf(sg, dpp<kQuadXor1>(sg));
        sg = fmaxf(sg, dpp<kQuadXor2>(sg));
        if constexpr (G == 8) sg = fmaxf(sg, dpp<kRowRor4>(sg));
        if (n == 0) sigma[(size_t)u * cap + t] = valid ? sg : -INFINITY;
        s2[tt][i] = valid ? part * sm2 : -INFINITY;
      }
    }

    // -- online softmax (log2 units) ------------------------------------------
    float mloc = s2[0][0];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s2[tt][i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__ballot(alpha != 1.0f)) {
      l_part *= alpha;
#pragma unroll
      for (int T = 0; T < NT; ++T) z_part[T] *= alpha;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
    }
    m_run = m_new;

    float p[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tt][i] = __builtin_amdgcn_exp2f(s2[tt][i] - m_new);
        l_part += p[tt][i];
      }

    // -- P.V operand: column (g, h) gets fp16(p * s_g,t); sum p*z on the VALU --
    half8 bp[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      u32x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v0 = (t0 + 4 * kb + r) < len;
        const bool v1 = (t0 + 16 + 4 * kb + r) < len;
        const uint32_t m0 = cur.vm[T][0][r], m1 = cur.vm[T][1][r];
        const float ps0 = v0 ? p[0][r] * lo_half(m0) : 0.f;
        const float ps1 = v1 ? p[1][r] * lo_half(m1) : 0.f;
        z_part[T] += (v0 ? p[0][r] * hi_half(m0) : 0.f) + (v1 ? p[1][r] * hi_half(m1) : 0.f);
        w[r] = pack_half2(ps0, ps1);
      }
      bp[T] = __builtin_bit_cast(half8, w);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      uint32_t y = cur.vc[nt];
      if constexpr (VB == 2) y = (y & 0xFFu) | ((y & 0xFF00u) << 8);
      const half8 a = unpack8<VB>(y);
      const int T = (G == 8) ? (nt >> 2) : 0;
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp[T], acc[nt], 0, 0, 0);
    }
    if (more) cur = nxt;
  }

  // ---- combine the 4 waves of the workgroup -----------------------------------
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    z_part[T] += __shfl_xor(z_part[T], 16);
    z_part[T] += __shfl_xor(z_part[T], 32);
  }
  __shared__ float s_m[4][G];
  __shared__ float s_l[4][G];
  __shared__ float s_acc[4][G][kHeadDim];
  if (kb == 0 && n < G) {
    s_m[wv][h] = m_run;
    s_l[wv][h] = l_part;
  }
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int g = (G == 8) ? (2 * T + (n >> 3)) : (n >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nt = 2 * g + j;
      // nt is lane dependent; select the accumulator without dynamic indexing
      floatx4 a = acc[0];
#pragma unroll
      for (int x = 1; x < 8; ++x)
        if (x == nt) a = acc[x];
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[wv][h][16 * nt + 4 * kb + i] = a[i] + z_part[T];
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < G * kHeadDim; e += 256) {
    const int hh = e / kHeadDim;
    const int c = e - hh * kHeadDim;
    float M = s_m[0][hh];
#pragma unroll
    for (int x = 1; x < 4; ++x) M = fmaxf(M, s_m[x][hh]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float f = __builtin_amdgcn_exp2f(s_m[x][hh] - M);
        a += f * s_acc[x][hh][c];
        l += f * s_l[x][hh];
      }
    }
    const size_t rec = ((size_t)b * Hq + (size_t)kvh * G + hh) * nsplit + split;
    pacc[rec * kHeadDim + c] = a;
    if (c == 0) {
      pm[rec] = M;
      pl[rec] = l;
    }
  }
}

template <int KB, int VB, int G>
hipError_t launch_t(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                    float* sigma, const Partials& p, int nsplit, int chunk, hipStream_t s) {
  dim3 grid(nsplit, L.batch * L.n_kv_heads);
  (void)hipGetLastError();  // report only this launch's status
  decode_approx_kernel<KB, VB, G><<<grid, 256, 0, s>>>(
      static_cast<const uint8_t*>(c.k_codes), static_cast<const uint8_t*>(c.v_codes), c.k_meta,
      c.v_meta, q, sigma, p.m, p.l, p.acc, len, L.n_q_heads, L.n_kv_heads, L.capacity, nsplit, chunk);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_g(const bkv_layout& L, const bkv_cache& c, const uint16_t* q, const SeqArg& len,
                    float* sigma, const Partials& p, int nsplit, int chunk, hipStream_t s) {
  const int G = L.n_q_heads / L.n_kv_heads;
  if (G == 4) return launch_t<KB, VB, 4>(L, c, q, len, sigma, p, nsplit, chunk, s);
  return launch_t<KB, VB, 8>(L, c, q, len, sigma, p, nsplit, chunk, s);
}

}  // namespace

hipError_t launch_decode_approx(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                                const SeqArg& len, int max_len, float* sigma, const Partials& p,
                                int nsplit, int chunk, hipStream_t s) {
  (void)max_len;
  if (L.k_bits == 4 && L.v_bits == 4) return launch_g<4, 4>(L, c, q, len, sigma, p, nsplit, chunk, s);
  if (L.k_bits == 4 && L.v_bits == 2) return launch_g<4, 2>(L, c, q, len, sigma, p, nsplit, chunk, s);
  if (L.k_bits == 3 && L.v_bits == 4) return launch_g<3, 4>(L, c, q, len, sigma, p, nsplit, chunk, s);
  return launch_g<3, 2>(L, c, q, len, sigma, p, nsplit, chunk, s);
}

}  // namespace bkv
