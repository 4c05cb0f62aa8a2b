// topk.hip -- per (b, kvh): the min(k, len) tokens with the largest selection
// score, ties to the lower index, written in ascending index order.
// (JetFire README, introduction: only the top-k tokens get the high-precision
// correction; Jet-QSparse abstract: the budget is per KV head.)
//
// Scores map to order-preserving 32-bit keys.  Two launches, each spread over
// `nslice` workgroups per unit so that the whole GPU reads the scores (the
// unit's histogram and control words were cleared by the scan that wrote the
// scores, earlier in the same step):
//   pass 1 histogram of the top 12 key bits (LDS per slice, then global
//          atomics); the last workgroup to finish finds the 12-bit digit d1
//          that holds the k-th largest key and the count above it;
//   pass 2 every slice writes a bitmap of the tokens whose digit is > d1 and
//          appends the tokens whose digit is == d1 (the candidates) to a list;
//          the last workgroup resolves the candidates exactly (a radix select
//          over the remaining 20 bits, then the lowest indices among the keys
//          equal to the k-th), sets their bits, and turns the bitmap into the
//          sorted index list.  If the candidates overflow the list (degenerate
//          score distributions) the last workgroup re-reads the unit's scores
//          for the remaining radix passes.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Cross-workgroup data of one launch moves only through agent-scope atomics,
// which are performed at the device's coherence point: no cache maintenance
// (a device-wide fence writes back and invalidates the L2 of every XCD) is
// needed.  A workgroup publishes by finishing all its memory operations
// (s_waitcnt 0 in every wave, then a barrier) before its arrival atomic.
__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory operation this wave issued has completed.
__device__ inline void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Arrival at a per-unit counter after publishing; true in the last of `count`.
__device__ inline bool arrive_last(uint32_t* counter, uint32_t count, int* s_flag) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = (atomicAdd(counter, 1u) == count - 1);
  __syncthreads();
  return *s_flag != 0;
}

// Exclusive prefix sum over the workgroup; `total` gets the sum of all.
__device__ inline int block_excl_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wv] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_tmp[w];
    before += (w < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Given an LDS histogram of nb bins, find the digit d holding the need-th
// largest element (counting from the top): count(digit > d) < need <=
// count(digit >= d).  Returns d and, through `above`, count(digit > d).
__device__ inline int find_digit(const uint32_t* hist, int nb, int need, int* s_tmp, int* s_res, int& above) {
  const int per = nb / kThreads;
  if (threadIdx.x == 0) {
    s_res[0] = 0;
    s_res[1] = 0;
  }
  int mine = 0;
  for (int j = 0; j < per; ++j) mine += (int)hist[nb - 1 - (threadIdx.x * per + j)];
  int total;
  const int before = block_excl_scan(mine, s_tmp, total);  // also orders the s_res reset
  if (before < need && before + mine >= need) {
    int run = before;
    for (int j = 0; j < per; ++j) {
      const int d = nb - 1 - (threadIdx.x * per + j);
      const int c = (int)hist[d];
      if (run + c >= need) {
        s_res[0] = d;
        s_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  above = s_res[1];
  const int d = s_res[0];
  __syncthreads();
  return d;
}

__global__ __launch_bounds__(kThreads) void topk_pass1_kernel(const float* __restrict__ sigma, TopkScratch tk,
                                                              SeqArg lens, int Hkv, int cap, int k, int slice) {
  const int u = blockIdx.y;
  const int n = lens.v[u / Hkv];
  const int kk = min(k, n);
  const int t_lo = blockIdx.x * slice;
  const int t_hi = min(n, t_lo + slice);
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_res[2];
  __shared__ int s_last;
  const bool work = kk > 0 && kk < n;  // otherwise the selection is trivial
  if (work) {
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) s_hist[i] = 0;
    __syncthreads();
    const float* sg = sigma + (size_t)u * cap;
    for (int base = t_lo; base < t_hi; base += 8 * kThreads) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = base + j * kThreads + threadIdx.x;
        v[j] = (t < t_hi) ? sg[t] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = base + j * kThreads + threadIdx.x;
        if (t < t_hi) atomicAdd(&s_hist[float_key(v[j]) >> 20], 1u);
      }
    }
    __syncthreads();
    uint32_t* gh = tk.hist + (size_t)u * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads)
      if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
  }
  uint32_t* ctrl = tk.ctrl + (size_t)u * kCtrlWords;
  if (!arrive_last(&ctrl[kCtlArrive1], gridDim.x, &s_last) || !work) return;
  const uint32_t* gh = tk.hist + (size_t)u * kHistBins;
  {
    uint32_t v[kHistBins / kThreads];
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j) v[j] = ld_dev(&gh[j * kThreads + threadIdx.x]);
#pragma unroll
    for (int j = 0; j < kHistBins / kThreads; ++j) s_hist[j * kThreads + threadIdx.x] = v[j];
  }
  __syncthreads();
  int above;
  const int d1 = find_digit(s_hist, kHistBins, kk, s_tmp, s_res, above);
  if (threadIdx.x == 0) {
    st_dev(&ctrl[kCtlDigit1], (uint32_t)d1);
    st_dev(&ctrl[kCtlAbove1], (uint32_t)above);
  }
}

// The last workgroup's exact resolution of the threshold bucket.  On return
// every selected candidate's bit is set in the unit's bitmap (global).
__device__ void resolve_candidates(const float* __restrict__ sg, uint32_t* __restrict__ bm, const uint32_t* ctrl,
                                   const uint64_t* __restrict__ cand, int n, int kk, uint32_t* s_key,
                                   uint32_t* s_idx, uint32_t* s_hist, int* s_tmp, int* s_res) {
  const uint32_t d1 = ld_dev(&ctrl[kCtlDigit1]);
  const int need1 = kk - (int)ld_dev(&ctrl[kCtlAbove1]);
  const int cc = (int)ld_dev(&ctrl[kCtlCandCount]);
  const bool in_lds = cc <= kCandCap;
  if (in_lds) {
    for (int i0 = 0; i0 < cc; i0 += 4 * kThreads) {
      uint64_t e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * kThreads + threadIdx.x;
        e[j] = i < cc ? ld_dev64(&cand[i]) : 0ull;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * kThreads + threadIdx.x;
        if (i < cc) {
          s_key[i] = (uint32_t)(e[j] >> 32);
          s_idx[i] = (uint32_t)e[j];
        }
      }
    }
    __syncthreads();
  }
  // two more radix digits (bits 19..10 and 9..0) among the bucket's keys
  uint32_t prefix = d1 << 20, pmask = 0xFFF00000u;
  int need = need1;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    for (int i = threadIdx.x; i < 1024; i += kThreads) s_hist[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (int i = threadIdx.x; i < cc; i += kThreads)
        if ((s_key[i] & pmask) == prefix) atomicAdd(&s_hist[(s_key[i] >> shift) & 1023u], 1u);
    } else {
      for (int t = threadIdx.x; t < n; t += kThreads) {
        const uint32_t key = float_key(sg[t]);
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 1023u], 1u);
      }
    }
    __syncthreads();
    int above;
    const int d = find_digit(s_hist, 1024, need, s_tmp, s_res, above);
    need -= above;
    prefix |= (uint32_t)d << shift;
    pmask |= 1023u << shift;
  }
  const uint32_t T = prefix;  // the k-th largest key; `need` keys equal to T are taken
  int te = 0;
  {
    int mine = 0;
    if (in_lds) {
      for (int i = threadIdx.x; i < cc; i += kThreads) mine += (s_key[i] == T);
    } else {
      for (int t = threadIdx.x; t < n; t += kThreads) mine += (float_key(sg[t]) == T);
    }
    block_excl_scan(mine, s_tmp, te);
  }
  // Among the keys equal to T the `need` lowest indices are taken: a radix
  // select of the need-th largest ~index (11 + 11 + 10 bits).
  uint32_t tie_lim = 0xFFFFFFFFu;  // ties with index <= tie_lim are taken
  if (te > need) {
    uint32_t tp = 0, tm = 0;
    int nd = need;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      for (int i = threadIdx.x; i < nb; i += kThreads) s_hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (int i = threadIdx.x; i < cc; i += kThreads)
          if (s_key[i] == T) {
            const uint32_t r = ~s_idx[i];
            if ((r & tm) == tp) atomicAdd(&s_hist[(r >> shift) & (uint32_t)(nb - 1)], 1u);
          }
      } else {
        for (int t = threadIdx.x; t < n; t += kThreads)
          if (float_key(sg[t]) == T) {
            const uint32_t r = ~(uint32_t)t;
            if ((r & tm) == tp) atomicAdd(&s_hist[(r >> shift) & (uint32_t)(nb - 1)], 1u);
          }
      }
      __syncthreads();
      int above;
      const int d = find_digit(s_hist, nb, nd, s_tmp, s_res, above);
      nd -= above;
      tp |= (uint32_t)d << shift;
      tm |= (uint32_t)(nb - 1) << shift;
    }
    tie_lim = ~tp;
  }
  if (in_lds) {
    for (int i = threadIdx.x; i < cc; i += kThreads) {
      const uint32_t key = s_key[i], t = s_idx[i];
      if (key > T || (key == T && t <= tie_lim)) atomicOr(&bm[t >> 5], 1u << (t & 31));
    }
  } else {
    for (int t = threadIdx.x; t < n; t += kThreads) {
      const uint32_t key = float_key(sg[t]);
      if ((key >> 20) == d1 && (key > T || (key == T && (uint32_t)t <= tie_lim)))
        atomicOr(&bm[t >> 5], 1u << (t & 31));
    }
  }
  wait_mem();
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_pass2_kernel(const float* __restrict__ sigma, TopkScratch tk,
                                                              int32_t* __restrict__ idx, SeqArg lens, int Hkv,
                                                              int cap, int k, int slice) {
  const int u = blockIdx.y;
  const int n = lens.v[u / Hkv];
  const int kk = min(k, n);
  const int t_lo = blockIdx.x * slice;
  const int t_hi = min(n, t_lo + slice);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const float* sg = sigma + (size_t)u * cap;
  uint32_t* ctrl = tk.ctrl + (size_t)u * kCtrlWords;
  uint32_t* bm = tk.bitmap + (size_t)u * (cap / 32);
  uint64_t* cand = tk.cand + (size_t)u * kCandCap;
  const bool resolve = kk > 0 && kk < n;
  const uint32_t d1 = resolve ? ctrl[kCtlDigit1] : 0u;

  // bitmap words of this slice (slices are multiples of 1024 tokens)
  for (int base0 = t_lo; base0 < t_hi; base0 += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = base0 + j * kThreads + threadIdx.x;
      v[j] = (resolve && t < t_hi) ? sg[t] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int base = base0 + j * kThreads;
      if (base >= t_hi) break;  // uniform
      const int t = base + threadIdx.x;
      bool bit = false;
      if (t < t_hi) {
        if (kk == n) {
          bit = true;
        } else if (resolve) {
          const uint32_t key = float_key(v[j]);
          bit = (key >> 20) > d1;
          if ((key >> 20) == d1) {
            // wave-aggregated append to the candidate list
            const uint64_t m = __ballot(true);
            const int nlead = __popcll(m & ((1ull << lane) - 1));
            uint32_t slot0 = 0;
            if (nlead == 0) slot0 = atomicAdd(&ctrl[kCtlCandCount], (uint32_t)__popcll(m));
            slot0 = __shfl(slot0, __ffsll((unsigned long long)m) - 1);
            const uint32_t slot = slot0 + nlead;
            if (slot < (uint32_t)kCandCap) st_dev64(&cand[slot], ((uint64_t)key << 32) | (uint32_t)t);
          }
        }
      }
      const uint64_t word = __ballot(bit);
      const int w0 = (base + wv * 64) >> 5;
      if (lane == 0 && base + wv * 64 < t_hi) st_dev(&bm[w0], (uint32_t)word);
      if (lane == 0 && base + wv * 64 + 32 < t_hi) st_dev(&bm[w0 + 1], (uint32_t)(word >> 32));
    }
  }
  __shared__ int s_last;
  if (!arrive_last(&ctrl[kCtlArrive2], gridDim.x, &s_last)) return;

  __shared__ uint32_t s_key[kCandCap];
  __shared__ uint32_t s_idx[kCandCap];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_res[2];
  if (resolve) resolve_candidates(sg, bm, ctrl, cand, n, kk, s_key, s_idx, s_hist, s_tmp, s_res);

  // bitmap -> ascending index list: thread j owns words [j*per, j*per+per)
  int32_t* out = idx + (size_t)u * k;
  const int nw = (n + 31) / 32;
  const int per = (nw + kThreads - 1) / kThreads;
  const int w_lo = threadIdx.x * per;
  int mine = 0;
  for (int w0 = 0; w0 < per; w0 += 8) {
    uint32_t b8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b8[j] = (w0 + j < per && w_lo + w0 + j < nw) ? ld_dev(&bm[w_lo + w0 + j]) : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) mine += __popc(b8[j]);
  }
  int total;
  int pos = block_excl_scan(mine, s_tmp, total);
  for (int w = w_lo; w < min(nw, w_lo + per); ++w) {
    uint32_t bits = ld_dev(&bm[w]);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < kk) out[pos] = w * 32 + b;
      ++pos;
    }
  }
  for (int i = kk + threadIdx.x; i < k; i += kThreads) out[i] = -1;
}

}  // namespace

int topk_slice(int units, int max_len) {
  // slices of whole 1024-token blocks, about 512 workgroups in all
  long long per = ((long long)units * (max_len > 0 ? max_len : 1) + 511) / 512;
  per = ((per + 1023) / 1024) * 1024;
  return per < 1024 ? 1024 : (int)per;
}

hipError_t launch_topk(const bkv_layout& L, const float* sigma, const SeqArg& len, int max_len, int k,
                       int32_t* idx, const TopkScratch& tk, hipStream_t s) {
  const int units = L.batch * L.n_kv_heads;
  const int slice = topk_slice(units, max_len);
  const int nslice = max(1, (max_len + slice - 1) / slice);
  (void)hipGetLastError();  // report only this call's launches
  topk_pass1_kernel<<<dim3(nslice, units), kThreads, 0, s>>>(sigma, tk, len, L.n_kv_heads, L.capacity, k, slice);
  topk_pass2_kernel<<<dim3(nslice, units), kThreads, 0, s>>>(sigma, tk, idx, len, L.n_kv_heads, L.capacity, k,
                                                             slice);
  return hipGetLastError();
}

}  // namespace bkv
