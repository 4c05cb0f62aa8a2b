// topk.hip -- per (b, kvh): the min(k, len) tokens with the largest selection
// score, ties to the lower index, written in ascending index order.
// (JetFire README, introduction: only the top-k tokens get the high-precision
// correction; Jet-QSparse abstract: the budget is per KV head.)
//
// One workgroup of 1024 threads per unit.  Scores map to order-preserving
// 32-bit keys; an MSB-first radix select with digits of 12, 10 and 10 bits
// (LDS histograms) finds the k-th largest key T and how many keys equal to T
// must be taken (r).  A final pass in index order takes every key > T and the
// first r keys == T, using wave ballots for the running ranks, so the output
// is sorted and deterministic.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = 4096;

__device__ inline int block_exclusive_scan(int v, int* s_wave, int& total) {
  // inclusive scan inside the wave by shuffles, then across waves via LDS
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_wave[w];
    before += (w < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ sigma,
                                                        int32_t* __restrict__ idx, SeqArg lens,
                                                        int Hkv, int cap, int k) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int n = lens.v[b];
  const int kk = min(k, n);
  const float* sg = sigma + (size_t)u * cap;
  int32_t* out = idx + (size_t)u * k;
  const int tid = threadIdx.x;

  for (int i = kk + tid; i < k; i += kThreads) out[i] = -1;
  if (kk == 0) return;
  if (kk == n) {  // everything is selected
    for (int i = tid; i < n; i += kThreads) out[i] = i;
    return;
  }

  __shared__ int hist[kMaxBins];
  __shared__ int s_wave[kWaves];
  __shared__ int s_sel[2];  // digit, count of keys above it

  uint32_t prefix = 0, pmask = 0;
  int need = kk;
  const int shifts[3] = {20, 10, 0};
  const int widths[3] = {12, 10, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    for (int i = tid; i < nb; i += kThreads) hist[i] = 0;
    if (tid == 0) {
      s_sel[0] = 0;
      s_sel[1] = 0;
    }
    __syncthreads();
    for (int t = tid; t < n; t += kThreads) {
      const uint32_t key = float_key(sg[t]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // Digits descend; thread j owns bins [nb-1-j*per, ...] counted from the top.
    const int per = nb / kThreads;  // 4 or 1
    int mine = 0;
    for (int j = 0; j < per; ++j) mine += hist[nb - 1 - (tid * per + j)];
    int total;
    const int above = block_exclusive_scan(mine, s_wave, total);  // keys in higher bins
    if (above < need && above + mine >= need) {
      int run = above;
      for (int j = 0; j < per; ++j) {
        const int d = nb - 1 - (tid * per + j);
        const int c = hist[d];
        if (run + c >= need) {
          s_sel[0] = d;
          s_sel[1] = run;
          break;
        }
        run += c;
      }
    }
    __syncthreads();
    const int digit = s_sel[0];
    need -= s_sel[1];
    prefix |= (uint32_t)digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the k-th largest key; take `need` of the keys equal to it

  int base_sel = 0, base_eq = 0;
  for (int t0 = 0; t0 < n; t0 += kThreads) {
    const int t = t0 + tid;
    uint32_t key = 0;
    if (t < n) key = float_key(sg[t]);
    const bool gt = (t < n) && key > T;
    const bool eq = (t < n) && key == T;
    int tot_eq;
    const int eq_rank = base_eq + block_exclusive_scan(eq ? 1 : 0, s_wave, tot_eq);
    const bool sel = gt || (eq && eq_rank < need);
    int tot_sel;
    const int pos = base_sel + block_exclusive_scan(sel ? 1 : 0, s_wave, tot_sel);
    if (sel && pos < kk) out[pos] = t;
    base_eq += tot_eq;
    base_sel += tot_sel;
  }
}

}  // namespace

hipError_t launch_topk(const bkv_layout& L, const float* sigma, const SeqArg& len, int k,
                       int32_t* idx, hipStream_t s) {
  (void)hipGetLastError();  // report only this launch's status
  topk_kernel<<<L.batch * L.n_kv_heads, kThreads, 0, s>>>(sigma, idx, len, L.n_kv_heads, L.capacity, k);
  return hipGetLastError();
}

}  // namespace bkv
