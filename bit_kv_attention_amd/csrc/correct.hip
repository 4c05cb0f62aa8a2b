// correct.hip -- merge the split softmax states and apply the exact correction
// to the selected tokens (JetFire README, introduction: the top-k tokens get a
// high-precision correction; here from the fp16 shadow rows).
//
// With the merged approximate state (M, L, A) of head h (log2 units, relative
// to M), the selected set S, exact logits s_t and approximate ones s_hat_t:
//   m' = max(M, max_S s_t)
//   l' = 2^(M-m') (L - sum_S 2^(s_hat_t - M))        + sum_S 2^(s_t - m')
//   a' = 2^(M-m') (A - sum_S 2^(s_hat_t - M) V_hat_t) + sum_S 2^(s_t - m') V_t
//   out = a' / l'
// i.e. the selected tokens' approximate terms are taken out of the sums and
// their exact terms put in, then everything is renormalised.  When every token
// is selected the approximate state is dropped altogether.
//
// One workgroup of 256 threads per (b, kvh) unit handles its G query heads;
// selected tokens go 32 at a time: 8 threads per token for the two logits of
// every head, then 2 x 128 threads (one per channel) for the value sums.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;

__device__ inline float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

template <int KB, int VB, int G>
__global__ __launch_bounds__(256) void correct_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const uint32_t* __restrict__ k_meta, const uint32_t* __restrict__ v_meta,
    const uint16_t* __restrict__ k_shadow, const uint16_t* __restrict__ v_shadow,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, const float* __restrict__ pm,
    const float* __restrict__ pl, const float* __restrict__ pacc, float* __restrict__ out,
    SeqArg lens, int Hq, int Hkv, int cap, int nsplit, int k) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int kvh = u - b * Hkv;
  const int n = lens.v[b];
  const int tid = threadIdx.x;
  const size_t head0 = (size_t)b * Hq + (size_t)kvh * G;
  float* o = out + head0 * kHeadDim;

  if (n == 0) {
    for (int e = tid; e < G * kHeadDim; e += 256) o[e] = 0.f;
    return;
  }
  const int kk = min(k, n);
  const bool all_selected = (kk == n);
  const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;

  __shared__ float s_q[G][kHeadDim];
  __shared__ float s_M[G], s_L[G], s_A[G][kHeadDim];
  __shared__ float s_ex[kChunk][G], s_ap[kChunk][G];
  __shared__ float s_wex[kChunk][G], s_wap[kChunk][G];
  __shared__ int s_t[kChunk];
  __shared__ float s_mex[G], s_resc[G], s_exl[G], s_apl[G];
  __shared__ float s_part[2][2][G][kHeadDim];

  for (int e = tid; e < G * kHeadDim; e += 256) s_q[e / kHeadDim][e % kHeadDim] = h2f(q[head0 * kHeadDim + e]);

  // ---- merge the split states ----------------------------------------------
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int h = e / kHeadDim, c = e % kHeadDim;
    const size_t rec0 = (head0 + h) * nsplit;
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, pm[rec0 + sp]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < nsplit; ++sp) {
        const float f = __builtin_amdgcn_exp2f(pm[rec0 + sp] - M);
        a += f * pacc[(rec0 + sp) * kHeadDim + c];
        l += f * pl[rec0 + sp];
      }
    }
    s_A[h][c] = a;
    if (c == 0) {
      s_M[h] = M;
      s_L[h] = l;
    }
  }
  if (tid < G) {
    s_mex[tid] = -INFINITY;
    s_exl[tid] = 0.f;
    s_apl[tid] = 0.f;
  }

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  const uint32_t* kmeta = k_meta + (size_t)u * kGroups * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * kGroups * cap;
  const uint16_t* ksh = k_shadow + (size_t)u * cap * kHeadDim;
  const uint16_t* vsh = v_shadow + (size_t)u * cap * kHeadDim;
  const int32_t* my_idx = idx + (size_t)u * k;

  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  float exa[G], apa[G];
#pragma unroll
  for (int h = 0; h < G; ++h) exa[h] = apa[h] = 0.f;
  __syncthreads();

  for (int cb = 0; cb < kk; cb += kChunk) {
    // ---- logits of up to 32 selected tokens: 8 threads per token ----------
    {
      const int tl = tid >> 3;
      const int part = tid & 7;
      const int ip = cb + tl;
      int t = (ip < kk) ? my_idx[ip] : -1;
      if (t >= n) t = -1;
      float ex[G], ap[G];
#pragma unroll
      for (int h = 0; h < G; ++h) ex[h] = ap[h] = 0.f;
      if (t >= 0) {
        const int c0 = 16 * part;
        const uint16_t* kr = ksh + (size_t)t * kHeadDim + c0;
        const uint32_t* row = reinterpret_cast<const uint32_t*>(kbase + (size_t)t * (kHeadDim * KB / 8));
        const int bit0 = c0 * KB;
        const int w0 = bit0 >> 5;
        const uint64_t bits = ((uint64_t)row[w0] | ((uint64_t)row[w0 + 1] << 32)) >> (bit0 & 31);
        const uint32_t mw = kmeta[(size_t)(c0 / kGroup) * cap + t];
        const float s = h2f((uint16_t)(mw & 0xFFFFu)), z = h2f((uint16_t)(mw >> 16));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float kx = h2f(kr[j]);
          const float kh = s * (float)((bits >> (KB * j)) & ((1u << KB) - 1)) + z;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            ex[h] += s_q[h][c0 + j] * kx;
            ap[h] += s_q[h][c0 + j] * kh;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
          ex[h] += __shfl_xor(ex[h], off);
          ap[h] += __shfl_xor(ap[h], off);
        }
      }
      if (part == 0) {
        s_t[tl] = t;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s_ex[tl][h] = (t >= 0) ? ex[h] * sm2 : -INFINITY;
          s_ap[tl][h] = (t >= 0) ? ap[h] * sm2 : -INFINITY;
        }
      }
    }
    __syncthreads();
    // ---- running max of the exact logits, weights ---------------------------
    if (tid < G) {
      float cm = -INFINITY;
      for (int tl = 0; tl < kChunk; ++tl) cm = fmaxf(cm, s_ex[tl][tid]);
      const float mold = s_mex[tid];
      const float mnew = fmaxf(mold, cm);
      s_resc[tid] = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mold - mnew);
      s_mex[tid] = mnew;
    }
    __syncthreads();
    {
      const int tl = tid >> 3;
      const int h = tid & 7;
      if (h < G) {
        const float mnew = s_mex[h];
        s_wex[tl][h] = (s_t[tl] >= 0) ? __builtin_amdgcn_exp2f(s_ex[tl][h] - mnew) : 0.f;
        s_wap[tl][h] = (s_t[tl] >= 0) ? __builtin_amdgcn_exp2f(s_ap[tl][h] - s_M[h]) : 0.f;
      }
    }
    __syncthreads();
    if (tid < G) {
      float el = 0.f, al = 0.f;
      for (int tl = 0; tl < kChunk; ++tl) {
        el += s_wex[tl][tid];
        al += s_wap[tl][tid];
      }
      s_exl[tid] = s_exl[tid] * s_resc[tid] + el;
      s_apl[tid] += al;
    }
    // ---- value sums: one thread per (channel, half of the chunk) -------------
#pragma unroll
    for (int h = 0; h < G; ++h) exa[h] *= s_resc[h];
    for (int tl = half * (kChunk / 2); tl < (half + 1) * (kChunk / 2); ++tl) {
      const int t = s_t[tl];
      if (t < 0) continue;
      const float v = h2f(vsh[(size_t)t * kHeadDim + c]);
      const int tile = t / kTile, r = t % kTile;
      const int qq = (r & 15) >> 2;
      const int slot = 4 * (r >> 4) + (r & 3);
      const uint8_t* vt = vbase + (size_t)tile * v_tile_bytes(VB);
      uint32_t code;
      if constexpr (VB == 4)
        code = (reinterpret_cast<const uint32_t*>(vt)[c * 4 + qq] >> (4 * slot)) & 15u;
      else
        code = (reinterpret_cast<const uint16_t*>(vt)[c * 4 + qq] >> (2 * slot)) & 3u;
      const uint32_t mw = vmeta[(size_t)(c / kGroup) * cap + t];
      const float vh = h2f((uint16_t)(mw & 0xFFFFu)) * (float)code + h2f((uint16_t)(mw >> 16));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        exa[h] += s_wex[tl][h] * v;
        apa[h] += s_wap[tl][h] * vh;
      }
    }
    __syncthreads();
  }

  // ---- combine the two halves and finish -------------------------------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_part[0][half][h][c] = exa[h];
    s_part[1][half][h][c] = apa[h];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int h = e / kHeadDim, cc = e % kHeadDim;
    const float ex_a = s_part[0][0][h][cc] + s_part[0][1][h][cc];
    const float ap_a = s_part[1][0][h][cc] + s_part[1][1][h][cc];
    const float M = s_M[h], mex = s_mex[h];
    float res;
    if (all_selected) {
      res = ex_a / s_exl[h];
    } else {
      const float mp = fmaxf(M, mex);
      const float fa = __builtin_amdgcn_exp2f(M - mp);
      const float fe = (mex == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mex - mp);
      const float l = fa * fmaxf(s_L[h] - s_apl[h], 0.f) + fe * s_exl[h];
      const float a = fa * (s_A[h][cc] - ap_a) + fe * ex_a;
      res = a / l;
    }
    o[(size_t)h * kHeadDim + cc] = res;
  }
}

template <int KB, int VB, int G>
hipError_t launch_t(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
                    const int32_t* idx, int k, const Partials& p, int nsplit, float* out, hipStream_t s) {
  (void)hipGetLastError();  // report only this launch's status
  correct_kernel<KB, VB, G><<<L.batch * L.n_kv_heads, 256, 0, s>>>(
      static_cast<const uint8_t*>(cc.k_codes), static_cast<const uint8_t*>(cc.v_codes), cc.k_meta,
      cc.v_meta, cc.k_shadow, cc.v_shadow, q, idx, p.m, p.l, p.acc, out, len, L.n_q_heads,
      L.n_kv_heads, L.capacity, nsplit, k);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_g(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
                    const int32_t* idx, int k, const Partials& p, int nsplit, float* out, hipStream_t s) {
  if (L.n_q_heads / L.n_kv_heads == 4) return launch_t<KB, VB, 4>(L, cc, q, len, idx, k, p, nsplit, out, s);
  return launch_t<KB, VB, 8>(L, cc, q, len, idx, k, p, nsplit, out, s);
}

}  // namespace

hipError_t launch_correct(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                          const SeqArg& len, const int32_t* idx, int k, const Partials& p,
                          int nsplit, float* out, hipStream_t s) {
  if (L.k_bits == 4 && L.v_bits == 4) return launch_g<4, 4>(L, c, q, len, idx, k, p, nsplit, out, s);
  if (L.k_bits == 4 && L.v_bits == 2) return launch_g<4, 2>(L, c, q, len, idx, k, p, nsplit, out, s);
  if (L.k_bits == 3 && L.v_bits == 4) return launch_g<3, 4>(L, c, q, len, idx, k, p, nsplit, out, s);
  return launch_g<3, 2>(L, c, q, len, idx, k, p, nsplit, out, s);
}

}  // namespace bkv
