// correct.hip -- exact correction of the selected tokens, then the merge of
// everything into the output (JetFire README, introduction: the top-k tokens
// get a high-precision correction; here from the fp16 shadow rows).
//
// With the merged approximate state (M, L, A) of head h over all tokens (log2
// units), the selected set S, exact logits s_t and approximate ones s_hat_t:
//   m' = max(M, max_S s_t)
//   l' = 2^(M-m') (L - sum_S 2^(s_hat_t - M))        + sum_S 2^(s_t - m')
//   a' = 2^(M-m') (A - sum_S 2^(s_hat_t - M) V_hat_t) + sum_S 2^(s_t - m') V_t
//   out = a' / l'
// i.e. the selected tokens' approximate terms leave the sums and their exact
// terms enter, then everything is renormalised.  When every token is selected
// the approximate state is not used at all.
//
// Two launches:
//   chunk   one workgroup per (unit, 32 selected tokens): exact and
//           approximate logits of the chunk's tokens for the unit's G query
//           heads (8 threads per token), then per head the chunk's exact state
//           (m, l, sum 2^(s-m) V) and approximate state (same with s_hat,
//           V_hat), one thread per channel for the value sums;
//   combine one workgroup per query head (one thread per channel): merges the
//           scan's split states and the chunk states as above.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

template <int KB, int VB, int G>
__global__ __launch_bounds__(256) void corr_chunk_kernel(
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ v_codes,
    const uint32_t* __restrict__ k_meta, const uint32_t* __restrict__ v_meta,
    const uint16_t* __restrict__ k_shadow, const uint16_t* __restrict__ v_shadow,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, float* __restrict__ cs,
    SeqArg lens, int Hq, int Hkv, int cap, int k, int nchunk) {
  const int u = blockIdx.y;
  const int chunk = blockIdx.x;
  const int b = u / Hkv;
  const int kvh = u - b * Hkv;
  const int n = lens.v[b];
  const int kk = min(k, n);
  const int ip0 = chunk * kCorrChunk;
  if (ip0 >= kk) return;  // the combine step reads only the chunks below kk
  const int tid = threadIdx.x;
  const size_t head0 = (size_t)b * Hq + (size_t)kvh * G;
  const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;

  __shared__ float s_q[G][kHeadDim];
  __shared__ int s_t[kCorrChunk];
  __shared__ float s_lg[2][kCorrChunk][G];  // logits, log2 units: [exact/approx]
  __shared__ float s_w[2][kCorrChunk][G];   // weights
  __shared__ float s_mx[2][G];
  __shared__ float s_part[2][2][G][kHeadDim];  // [exact/approx][half][h][c]

  if (tid < G * kHeadDim / 8) {
    const uint4 w = reinterpret_cast<const uint4*>(q + head0 * kHeadDim)[tid];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float* dst = &s_q[0][0] + tid * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[2 * j] = h2f((uint16_t)(ww[j] & 0xFFFFu));
      dst[2 * j + 1] = h2f((uint16_t)(ww[j] >> 16));
    }
  }
  if (tid < kCorrChunk) {
    int t = (ip0 + tid < kk) ? idx[(size_t)u * k + ip0 + tid] : -1;
    s_t[tid] = (t >= 0 && t < n) ? t : -1;
  }
  __syncthreads();

  const uint8_t* kbase = k_codes + (size_t)u * k_unit_bytes(KB, cap);
  const uint8_t* vbase = v_codes + (size_t)u * v_unit_bytes(VB, cap);
  const uint32_t* kmeta = k_meta + (size_t)u * kGroups * cap;
  const uint32_t* vmeta = v_meta + (size_t)u * kGroups * cap;
  const uint16_t* ksh = k_shadow + (size_t)u * cap * kHeadDim;
  const uint16_t* vsh = v_shadow + (size_t)u * cap * kHeadDim;

  // ---- logits: 8 threads per token, 16 channels each ------------------------
  {
    const int tl = tid >> 3;
    const int part = tid & 7;
    const int t = s_t[tl];
    float ex[G], ap[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ex[h] = ap[h] = 0.f;
    if (t >= 0) {
      const int c0 = 16 * part;
      const uint4* kr = reinterpret_cast<const uint4*>(ksh + (size_t)t * kHeadDim + c0);
      const uint4 k0 = kr[0], k1 = kr[1];
      const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      // channels c0..c0+15 are the group-(part/2) fields of the chunks of
      // eighths 2*(part%2) and 2*(part%2)+1 (8*KB bits each)
      uint32_t fld[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t* ch =
            reinterpret_cast<const uint32_t*>(kbase + k_chunk_offset(KB, t, 2 * (part & 1) + x));
        const int b0 = 8 * KB * (part >> 1);
        const int d0 = b0 >> 5, d1 = min(d0 + 1, KB - 1);
        fld[x] = (uint32_t)((((uint64_t)ch[d1] << 32) | ch[d0]) >> (b0 & 31));
      }
      const uint64_t bits = ((uint64_t)fld[0] & ((1ull << (8 * KB)) - 1)) | ((uint64_t)fld[1] << (8 * KB));
      const uint32_t mw = kmeta[(size_t)(c0 / kGroup) * cap + t];
      const float s = h2f((uint16_t)(mw & 0xFFFFu)), z = h2f((uint16_t)(mw >> 16));
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float kx = h2f((uint16_t)(kw[j >> 1] >> (16 * (j & 1))));
        const float kh = fmaf(s, (float)((bits >> (KB * j)) & ((1u << KB) - 1)), z);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          ex[h] = fmaf(s_q[h][c0 + j], kx, ex[h]);
          ap[h] = fmaf(s_q[h][c0 + j], kh, ap[h]);
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
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_lg[0][tl][h] = (t >= 0) ? ex[h] * sm2 : -INFINITY;
        s_lg[1][tl][h] = (t >= 0) ? ap[h] * sm2 : -INFINITY;
      }
    }
  }
  __syncthreads();
  if (tid < 2 * G) {
    const int ty = tid / G, h = tid % G;
    float m = -INFINITY;
    for (int tl = 0; tl < kCorrChunk; ++tl) m = fmaxf(m, s_lg[ty][tl][h]);
    s_mx[ty][h] = m;
  }
  __syncthreads();
  {
    const int tl = tid >> 3, h = tid & 7;
    if (h < G) {
      const bool ok = s_t[tl] >= 0;
      s_w[0][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[0][tl][h] - s_mx[0][h]) : 0.f;
      s_w[1][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[1][tl][h] - s_mx[1][h]) : 0.f;
    }
  }
  __syncthreads();

  // ---- value sums: one thread per (channel, half of the chunk) ---------------
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  float ea[G], aa[G];
#pragma unroll
  for (int h = 0; h < G; ++h) ea[h] = aa[h] = 0.f;
  constexpr int kHalf = kCorrChunk / 2;
  float vx[kHalf], vq[kHalf];
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {  // issue every load of the half chunk first
    const int t = s_t[half * kHalf + j];
    vx[j] = 0.f;
    vq[j] = 0.f;
    if (t >= 0) {
      int dw, bit;
      v_code_pos(VB, t % kTile, c, dw, bit);
      const uint32_t* vt = reinterpret_cast<const uint32_t*>(vbase + (size_t)(t / kTile) * v_tile_bytes(VB));
      const uint32_t code = (vt[dw] >> bit) & ((1u << VB) - 1);
      const uint32_t mw = vmeta[(size_t)(c / kGroup) * cap + t];
      vx[j] = h2f(vsh[(size_t)t * kHeadDim + c]);
      vq[j] = fmaf(h2f((uint16_t)(mw & 0xFFFFu)), (float)code, h2f((uint16_t)(mw >> 16)));
    }
  }
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    const int tl = half * kHalf + j;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ea[h] = fmaf(s_w[0][tl][h], vx[j], ea[h]);
      aa[h] = fmaf(s_w[1][tl][h], vq[j], aa[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s_part[0][half][h][c] = ea[h];
    s_part[1][half][h][c] = aa[h];
  }
  __syncthreads();
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int h = e / kHeadDim, cc = e % kHeadDim;
    float* rec = cs + ((head0 + h) * nchunk + chunk) * kCsStride;
    rec[4 + cc] = s_part[0][0][h][cc] + s_part[0][1][h][cc];
    rec[4 + kHeadDim + cc] = s_part[1][0][h][cc] + s_part[1][1][h][cc];
  }
  if (tid < 2 * G) {
    const int ty = tid / G, h = tid % G;
    float l = 0.f;
    for (int tl = 0; tl < kCorrChunk; ++tl) l += s_w[ty][tl][h];
    float* rec = cs + ((head0 + h) * nchunk + chunk) * kCsStride;
    rec[2 * ty] = s_mx[ty][h];
    rec[2 * ty + 1] = l;
  }
}

// One workgroup per query head, one thread per channel.  The per-split and
// per-chunk weights go through LDS in batches so that every channel thread
// only streams its accumulators.
constexpr int kBatchLds = 512;

__device__ inline float block_max128(float v, float* s_red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(s_red[0], s_red[1]);
}

__device__ inline float block_sum128(float v, float* s_red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return s_red[0] + s_red[1];
}

// sum over records j < cnt of w_j * rec_j[c], with w_j = 2^(m_j - ref) and
// m_j = rec_j[-moff]; also returns sum_j w_j * l_j (l_j = rec_j[loff - moff]).
__device__ inline void weighted_sums(const float* __restrict__ mbase, const float* __restrict__ lbase,
                                     const float* __restrict__ vbase, int stride_ml, int stride_v, int cnt,
                                     float ref, float* s_w, float* s_red, float& acc, float& lsum) {
  const int c = threadIdx.x;
  acc = 0.f;
  float lpart = 0.f;
  for (int j0 = 0; j0 < cnt; j0 += kBatchLds) {
    const int nb = min(kBatchLds, cnt - j0);
    __syncthreads();
    for (int j = c; j < nb; j += kHeadDim) {
      const float f = __builtin_amdgcn_exp2f(mbase[(size_t)(j0 + j) * stride_ml] - ref);
      s_w[j] = f;
      lpart = fmaf(f, lbase[(size_t)(j0 + j) * stride_ml], lpart);
    }
    __syncthreads();
    for (int j1 = 0; j1 < nb; j1 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (j1 + j < nb) ? vbase[(size_t)(j0 + j1 + j) * stride_v + c] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j1 + j < nb) acc = fmaf(s_w[j1 + j], v[j], acc);
    }
  }
  lsum = block_sum128(lpart, s_red);
}

__global__ __launch_bounds__(kHeadDim) void combine_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                           const float* __restrict__ pacc, const float* __restrict__ cs,
                                                           float* __restrict__ out, SeqArg lens, int Hq, int nsplit,
                                                           int nchunk, int k) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int c = threadIdx.x;
  const int n = lens.v[b];
  const size_t rec = (size_t)b * Hq + h;
  float* o = out + rec * kHeadDim;
  if (n == 0) {
    o[c] = 0.f;
    return;
  }
  const int kk = min(k, n);
  const int nc = (kk + kCorrChunk - 1) / kCorrChunk;
  const float* ps = cs + rec * nchunk * kCsStride;
  __shared__ float s_w[kBatchLds];
  __shared__ float s_red[2];

  // exact state of the selected tokens
  float me = -INFINITY;
  for (int j = c; j < nc; j += kHeadDim) me = fmaxf(me, ps[(size_t)j * kCsStride]);
  me = block_max128(me, s_red);
  float ae = 0.f, le = 0.f;
  if (nc > 0) weighted_sums(ps, ps + 1, ps + 4, kCsStride, kCsStride, nc, me, s_w, s_red, ae, le);
  if (kk == n) {
    o[c] = ae / le;
    return;
  }
  // approximate state of every token
  const float* sm = pm + rec * nsplit;
  float M = -INFINITY;
  for (int j = c; j < nsplit; j += kHeadDim) M = fmaxf(M, sm[j]);
  M = block_max128(M, s_red);
  float A, L;
  weighted_sums(sm, pl + rec * nsplit, pacc + rec * nsplit * kHeadDim, 1, kHeadDim, nsplit, M, s_w, s_red, A, L);
  if (kk == 0) {
    o[c] = A / L;
    return;
  }
  // the selected tokens' approximate terms, relative to M
  float as, ls;
  weighted_sums(ps + 2, ps + 3, ps + 4 + kHeadDim, kCsStride, kCsStride, nc, M, s_w, s_red, as, ls);
  const float mp = fmaxf(M, me);
  const float fa = __builtin_amdgcn_exp2f(M - mp);
  const float fe = __builtin_amdgcn_exp2f(me - mp);
  const float l = fa * fmaxf(L - ls, 0.f) + fe * le;
  const float a = fa * (A - as) + fe * ae;
  o[c] = a / l;
}

template <int KB, int VB, int G>
void launch_chunks(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
                   const int32_t* idx, int k, const Workspace& w, hipStream_t s) {
  corr_chunk_kernel<KB, VB, G><<<dim3(w.nchunk, L.batch * L.n_kv_heads), 256, 0, s>>>(
      static_cast<const uint8_t*>(cc.k_codes), static_cast<const uint8_t*>(cc.v_codes), cc.k_meta,
      cc.v_meta, cc.k_shadow, cc.v_shadow, q, idx, w.cs, len, L.n_q_heads, L.n_kv_heads, L.capacity, k,
      w.nchunk);
}

template <int KB, int VB>
void launch_chunks_g(const bkv_layout& L, const bkv_cache& cc, const uint16_t* q, const SeqArg& len,
                     const int32_t* idx, int k, const Workspace& w, hipStream_t s) {
  if (L.n_q_heads / L.n_kv_heads == 4)
    launch_chunks<KB, VB, 4>(L, cc, q, len, idx, k, w, s);
  else
    launch_chunks<KB, VB, 8>(L, cc, q, len, idx, k, w, s);
}

}  // namespace

hipError_t launch_correct(const bkv_layout& L, const bkv_cache& c, const uint16_t* q,
                          const SeqArg& len, const int32_t* idx, int k, const Workspace& w,
                          float* out, hipStream_t s) {
  (void)hipGetLastError();  // report only this call's launches
  if (w.nchunk > 0) {
    if (L.k_bits == 4 && L.v_bits == 4) launch_chunks_g<4, 4>(L, c, q, len, idx, k, w, s);
    else if (L.k_bits == 4 && L.v_bits == 2) launch_chunks_g<4, 2>(L, c, q, len, idx, k, w, s);
    else if (L.k_bits == 3 && L.v_bits == 4) launch_chunks_g<3, 4>(L, c, q, len, idx, k, w, s);
    else launch_chunks_g<3, 2>(L, c, q, len, idx, k, w, s);
  }
  combine_kernel<<<dim3(L.n_q_heads, L.batch), kHeadDim, 0, s>>>(w.part.m, w.part.l, w.part.acc, w.cs, out, len,
                                                                 L.n_q_heads, w.nsplit, w.nchunk, k);
  return hipGetLastError();
}

}  // namespace bkv
