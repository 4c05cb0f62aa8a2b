// select_lds.h -- the radix select on composite (score, index) keys shared by
// the top-k kernels and the fused select-and-correct kernel.
//
// A token's composite key is (order-preserving bits of its score) << 32 | ~t:
// larger means a larger score, or an equal score and a lower index, and no
// two tokens share one.  The need-th largest composite T is found most
// significant digit first (widths 12, 10, 10 over the score bits, 11, 11, 10
// over the index bits): a pass histograms the next digit of the entries under
// the prefix so far (LDS atomics), the digit holding the need-th largest is
// appended, and it stops once every entry under the prefix is needed; T is
// then the smallest composite with that prefix.
#pragma once

#include "bkv_internal.h"

namespace bkv {

constexpr int kLevels = 6;
__constant__ const int kDigitBits[kLevels] = {12, 10, 10, 11, 11, 10};

__device__ inline uint64_t composite(float s, int t) {
  return ((uint64_t)float_key(s) << 32) | (uint64_t)(~(uint32_t)t);
}

// Exclusive prefix sum over a workgroup of NW waves (wave shuffles, then the
// wave totals through LDS); `total` gets the sum of all.
template <int NW>
__device__ inline int block_excl_scan(int v, int* s_wsum, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) s_wsum[wv] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = s_wsum[w];
    before += (w < wv) ? s : 0;
    total += s;
  }
  return before + x - v;
}

// The need-th largest of `count` composites that LDS holds (get(i) gives
// entry i; entries equal to 0 are empty slots and never selected), by the
// radix select described above, entirely in LDS.  Returns T with exactly
// `need` entries >= T.  NT threads.
template <int NT, typename Get>
__device__ inline uint64_t lds_threshold(Get get, int count, int need, uint32_t* s_hist, int* s_wsum, int* s_res) {
  const int tid = threadIdx.x;
  uint64_t P = 0;
  int plen = 0;
  for (int lv = 0; lv < kLevels; ++lv) {
    const int d = kDigitBits[lv];
    const int nb = 1 << d;
    const int shift = 64 - plen - d;
    for (int i = tid; i < nb; i += NT) s_hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < count; i += NT) {
      const uint64_t c = get(i);
      if (plen == 0 || (c >> (64 - plen)) == P) atomicAdd(&s_hist[(uint32_t)(c >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int per = nb / NT;
    const int top = nb - 1 - tid * per;
    int mine = 0;
    for (int i = 0; i < per; ++i) mine += (int)s_hist[top - i];
    int total;
    int above = block_excl_scan<NT / 64>(mine, s_wsum, total);
    if (above < need && above + mine >= need) {
      for (int i = 0; i < per; ++i) {
        const int h = (int)s_hist[top - i];
        if (above + h >= need) {
          s_res[0] = top - i;
          s_res[1] = above;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
    const int D = s_res[0];
    need -= s_res[1];
    P = (P << d) | (uint64_t)D;
    plen += d;
    const int m = (int)s_hist[D];
    __syncthreads();
    if (m == need) break;
  }
  return (plen >= 64) ? P : (P << (64 - plen));
}

}  // namespace bkv
