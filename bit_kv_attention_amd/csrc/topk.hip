// topk.hip -- per (b, kvh): the min(k, len) tokens with the largest selection
// score, ties to the lower index, written in ascending index order.
// (JetFire README, introduction: only the top-k tokens get the high-precision
// correction; Jet-QSparse abstract: the budget is per KV head.)
// With a recent window of W tokens (HACK review and TailorKV review: the
// newest tokens are kept at full precision) the last nw = min(W, len) tokens
// are always taken: the selection runs over the first n = len - nw tokens,
// and a unit's row of k + W entries holds the min(k, n) selected indices,
// then n .. n + nw - 1, then -1.
//
// One workgroup of 1024 threads per unit; nothing leaves the workgroup until
// the answer is known, so there is no cross-workgroup protocol at all.
//
// Every token gets the composite key c(t) = (ordered bits of sigma_t) << 32 |
// ~t: larger c means a larger score, or an equal score and a lower index, and
// no two tokens share a c.  The selected set is {t : c(t) >= T} with T the
// kk-th largest composite, found by a radix select, most significant digit
// first (digit widths 12, 10, 10 over the score bits, 11, 11, 10 over the
// index bits):
//   a pass histograms the next digit of the entries that match the prefix so
//   far (LDS atomics), and the digit holding the kk-th largest is appended to
//   the prefix.  The first passes read the scores from memory; as soon as the
//   prefix matches at most kCandMax tokens those are copied into LDS and the
//   remaining passes run there.  It stops when every entry under the prefix
//   is needed; T is then the smallest composite with that prefix.
// Last, c(t) >= T becomes ascending indices: each wave owns a contiguous run
// of the tokens, counts its selected ones with ballots, a prefix sum over the
// 16 wave counts places the runs, and a second pass writes them in order.
#include "bkv_internal.h"
#include "select_lds.h"

namespace bkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCandMax = 4096;
constexpr int kBatch = 16;  // scores per thread loaded together (independent loads in flight)

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ sigma, int32_t* __restrict__ idx,
                                                        SeqArg lens, int Hkv, int cap, int k, int W) {
  const int u = blockIdx.x;
  const int b = u / Hkv;
  const int nw = min(W, lens.v[b]);
  const int n = lens.v[b] - nw;  // tokens to select from
  const int kk = min(k, n);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* __restrict__ sg = sigma + (size_t)u * cap;
  int32_t* __restrict__ out = idx + (size_t)u * (k + W);

  write_tail<kThreads>(out, kk, n, nw, k + W);
  if (kk == n || kk == 0) {  // every token (or none) is selected
    for (int i = tid; i < kk; i += kThreads) out[i] = i;
    return;
  }

  __shared__ uint32_t s_hist[1 << 12];
  __shared__ uint64_t s_cand[kCandMax];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_ncand;
  __shared__ int s_digit, s_above;

  uint64_t P = 0;  // prefix of T, plen bits
  int plen = 0;
  int need = kk;   // entries still to take under the prefix
  bool in_lds = false;
  int ncand = 0;

  for (int lv = 0; lv < kLevels; ++lv) {
    const int d = kDigitBits[lv];
    const int nb = 1 << d;
    const int shift = 64 - plen - d;
    for (int i = tid; i < nb; i += kThreads) s_hist[i] = 0u;
    __syncthreads();
    auto count = [&](uint64_t c) {
      if (plen == 0 || (c >> (64 - plen)) == P) atomicAdd(&s_hist[(uint32_t)(c >> shift) & (nb - 1)], 1u);
    };
    if (in_lds) {
      for (int i = tid; i < ncand; i += kThreads) count(s_cand[i]);
    } else {
      for (int t0 = 0; t0 < n; t0 += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int t = t0 + i * kThreads + tid;
          v[i] = sg[min(t, n - 1)];  // clamped: every load unconditional
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int t = t0 + i * kThreads + tid;
          if (t < n) count(composite(v[i], t));
        }
      }
    }
    __syncthreads();
    // the digit D with  sum_{x > D} hist[x] < need <= sum_{x >= D} hist[x]:
    // thread j owns the bins from nb-1-j*per downwards, per = nb / 1024
    const int per = nb / kThreads;
    const int top = nb - 1 - tid * per;
    int mine = 0;
    for (int i = 0; i < per; ++i) mine += (int)s_hist[top - i];
    int total;
    int above = block_excl_scan<kWaves>(mine, s_wsum, total);  // count in the bins above this thread's
    if (above < need && above + mine >= need) {
      for (int i = 0; i < per; ++i) {
        const int h = (int)s_hist[top - i];
        if (above + h >= need) {
          s_digit = top - i;
          s_above = above;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
    const int D = s_digit;
    need -= s_above;
    P = (P << d) | (uint64_t)D;
    plen += d;
    const int m = (int)s_hist[D];
    __syncthreads();  // everyone has read s_digit, s_above and s_hist
    if (m == need) break;
    if (!in_lds && m <= kCandMax) {
      // copy the tokens under the prefix into LDS (one LDS atomic per wave)
      if (tid == 0) s_ncand = 0;
      __syncthreads();
      for (int t0 = 0; t0 < n; t0 += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int t = t0 + i * kThreads + tid;
          v[i] = sg[min(t, n - 1)];  // clamped: every load unconditional
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int t = t0 + i * kThreads + tid;
          uint64_t c = 0;
          bool hit = false;
          if (t < n) {
            c = composite(v[i], t);
            hit = (c >> (64 - plen)) == P;
          }
          const uint64_t mask = __ballot(hit);
          if (mask) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&s_ncand, __popcll(mask));
            base = __shfl(base, 0);
            if (hit) s_cand[base + __popcll(mask & ((1ull << lane) - 1))] = c;
          }
        }
      }
      __syncthreads();
      in_lds = true;
      ncand = m;
    }
  }
  const uint64_t T = (plen >= 64) ? P : (P << (64 - plen));

  // ascending indices of {t : c(t) >= T}: wave w owns the contiguous range
  // [w*R, w*R + R) of 64-token blocks; it counts its selected tokens (ballot
  // popcounts), one prefix sum over the 16 wave counts places the ranges, and
  // the wave writes its tokens in order in a second pass.
  const int wv = tid >> 6;
  const int nblk = (n + 63) / 64;
  const int R = (nblk + kWaves - 1) / kWaves;  // blocks per wave
  const int b_lo = wv * R, b_hi = min(nblk, b_lo + R);
  auto sel_mask = [&](int blk, float v) -> uint64_t {
    const int t = blk * 64 + lane;
    return __ballot(t < n && composite(v, t) >= T);
  };
  int mine = 0;
  for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int t = (b0 + i) * 64 + lane;
      v[i] = sg[min(t, n - 1)];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (b0 + i < b_hi) mine += __popcll(sel_mask(b0 + i, v[i]));
  }
  int total;
  int pos = __shfl(block_excl_scan<kWaves>(lane == 0 ? mine : 0, s_wsum, total), 0);
  for (int b0 = b_lo; b0 < b_hi; b0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int t = (b0 + i) * 64 + lane;
      v[i] = sg[min(t, n - 1)];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (b0 + i < b_hi) {
        const uint64_t mask = sel_mask(b0 + i, v[i]);
        if ((mask >> lane) & 1ull) out[pos + __popcll(mask & ((1ull << lane) - 1))] = (b0 + i) * 64 + lane;
        pos += __popcll(mask);
      }
    }
  }
}

// ---- slice-local top-k, then the merge by the unit's last workgroup ---------
// Workgroup (slice s, unit) keeps the scores of tokens [s*S, s*S + S)
// (S <= kTopkSliceMax, chosen on the host) in LDS, finds the exact top
// min(kk, slice length) of the slice and writes their composites in index
// order to cand[u][s*k + j], and 0 into its slots past them.
// Every token of the unit's top-kk is in its slice's top-kk, so the union
// holds the answer.  Then it arrives at the unit's counter; the last of the
// unit's workgroups loads the nslice*k candidate slots into LDS (empty slots
// as 0), finds the kk-th largest composite T there and writes the candidates
// >= T in slot order, which is ascending token order, then clears the counter.
// Candidates cross workgroups through agent-scope atomic stores and loads,
// handed over by the arrival of select_lds.h (arrive_is_last).
constexpr int kLocalThreads = kThreads;
constexpr int kLocalMax = kTopkSliceMax;   // slice tokens in LDS
constexpr int kMergeMax = kTopkMergeMax;   // candidate slots in LDS per unit

template <bool FUSED>
__global__ __launch_bounds__(kLocalThreads) void topk_slices_kernel(const float* __restrict__ sigma,
                                                                    uint64_t* __restrict__ cand,
                                                                    uint32_t* __restrict__ counter,
                                                                    int32_t* __restrict__ idx, SeqArg lens, int Hkv,
                                                                    int cap, int k, int W, int S, int cstride) {
  __shared__ __attribute__((aligned(16))) float s_v[kLocalMax];  // the slice's scores; then (fused) the slots
  __shared__ uint32_t s_hist[1 << 12];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_res[4];
  __shared__ int s_last;
  __shared__ float s_mm[2 * kWaves];
  __shared__ uint64_t s_small[65];
  const int s = blockIdx.x, u = blockIdx.y;
  const int nw = min(W, lens.v[u / Hkv]);
  const int n = lens.v[u / Hkv] - nw;  // tokens to select from
  const int kk = min(k, n);
  const int t0 = s * S;
  const int len = min(S, n - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint64_t* __restrict__ ucand = cand + (size_t)u * cstride;

  if (0 < kk && kk < n && len > 0) {  // a slice with tokens to choose from
    const int cnt = min(kk, len);
    const float* __restrict__ sg = sigma + (size_t)u * cap + t0;
    // thread tid holds the contiguous tokens t0 + [tid*kPer, tid*kPer + kPer)
    constexpr int kPer = kLocalMax / kLocalThreads;
    const int i0 = tid * kPer;
    float v[kPer];
    if (i0 + kPer <= len) {
#pragma unroll
      for (int j = 0; j < kPer; j += 4) {
        const float4 x = *reinterpret_cast<const float4*>(sg + i0 + j);
        v[j] = x.x;
        v[j + 1] = x.y;
        v[j + 2] = x.z;
        v[j + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) v[j] = sg[min(i0 + j, len - 1)];  // clamped: unconditional
    }
    uint64_t c[kPer];  // 0: past the slice
#pragma unroll
    for (int j = 0; j < kPer; ++j) c[j] = (i0 + j < len) ? composite(v[j], t0 + i0 + j) : 0ull;
    auto get = [&](int i) { return composite(s_v[i], t0 + i); };
    auto fill = [&]() {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (i0 + j < len) s_v[i0 + j] = v[j];
    };
    const uint64_t T = (cnt == len) ? 0
                                    : hist_select<kLocalThreads>(c, len, cnt, get, fill, s_hist, s_wsum, s_res, s_mm,
                                                                 s_small);
    // the slice's entries >= T in index order
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += (c[j] && c[j] >= T) ? 1 : 0;
    int total;
    int pos = block_excl_scan<kWaves>(mine, s_wsum, total);
    uint64_t* __restrict__ dst = ucand + (size_t)s * k;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (c[j] && c[j] >= T) {
        if (FUSED) st_dev64(&dst[pos], c[j]); else dst[pos] = c[j];
        ++pos;
      }
    }
    for (int j = cnt + tid; j < k; j += kLocalThreads) {  // the slice's unused slots
      if (FUSED) st_dev64(&dst[j], 0ull); else dst[j] = 0ull;
    }
  }

  if (!FUSED) return;
  // ---- arrival; the unit's last workgroup merges ------------------------------
  if (!arrive_is_last(&counter[u], gridDim.x, &s_last)) return;

  merge_unit<kThreads, true, kLocalMax * 4 / 8>(ucand, idx, u, n, nw, k, W, S, reinterpret_cast<uint64_t*>(s_v), s_hist,
                                      s_wsum, s_res, s_mm, s_small);
  if (tid == 0) counter[u] = 0u;  // ready for the next call on this workspace
}

// The merge as a launch of its own (candidate slots beyond the slice stage's
// LDS footprint): one workgroup per unit.
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const uint64_t* __restrict__ cand,
                                                              int32_t* __restrict__ idx, SeqArg lens, int Hkv, int k,
                                                              int W, int S, int cstride) {
  __shared__ uint64_t s_c[kMergeMax];
  __shared__ uint32_t s_hist[1 << 12];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_res[4];
  __shared__ float s_mm[2 * kWaves];
  __shared__ uint64_t s_small[65];
  const int u = blockIdx.x;
  const int nw = min(W, lens.v[u / Hkv]);
  merge_unit<kThreads, false, kMergeMax>(cand + (size_t)u * cstride, idx, u, lens.v[u / Hkv] - nw, nw, k, W, S, s_c, s_hist,
                               s_wsum, s_res, s_mm, s_small);
}

// ---- block selection -----------------------------------------------------
// Block j holds tokens [j*bs, min(n, j*bs + bs)) and scores the largest sigma
// among them (Jet-QSparse abstract: the dense scan's scores choose whole
// 128-token blocks per KV head).  Workgroup (slice s, unit) reads the scores
// of tokens [s*kBlkSpan, s*kBlkSpan + kBlkSpan) with coalesced 16-byte loads
// (a wave covers 256 contiguous tokens per load, bs/4 lanes per block reduce
// by butterfly shuffles; a block longer than 256 tokens takes several loads
// of one wave) and stores its blocks' keys with agent-scope stores; the
// unit's last workgroup to arrive loads all nblk keys into LDS, finds the
// kb-th largest (score, block) composite as the token top-k does, ranks the
// chosen blocks in ascending order and writes the row as their tokens, block
// r at [r*bs, r*bs + bs), -1 past n.
constexpr int kBlkMax = kTopkBlocksMax;
constexpr int kBlkPer = kBlkMax / kThreads;
constexpr int kBlkBatch = 4;  // spans per wave with loads in flight together
constexpr int kBlkSpan = kTopkBlockSpan;  // tokens per workgroup (a multiple of every block size)


__global__ __launch_bounds__(kThreads) void topk_blocks_kernel(const float* __restrict__ sigma,
                                                               int32_t* __restrict__ idx, SeqArg lens, int Hkv,
                                                               int cap, int nb, int lgb, uint32_t* __restrict__ bkeys,
                                                               int kstride, uint32_t* __restrict__ counter) {
  __shared__ uint32_t s_bkey[kBlkMax];  // float_key of each block's largest score; then the chosen blocks
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_res[4];
  __shared__ int s_last;
  __shared__ float s_mm[2 * kWaves];
  __shared__ uint64_t s_small[65];
  const int sl = blockIdx.x, u = blockIdx.y;
  const int n = lens.v[u / Hkv];
  const int bs = 1 << lgb;
  const int nblk = (n + bs - 1) >> lgb;
  const int kb = min(nb, nblk);
  const int row = nb << lgb;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* __restrict__ out = idx + (size_t)u * row;
  if (kb == nblk) {  // every block (or none): the tokens in order, by the first slice; nothing arrives
    if (sl == 0)
      for (int i = tid; i < row; i += kThreads) out[i] = (i < n) ? i : -1;
    return;
  }

  // block maxima of this slice: wave wv takes spans of max(bs, 256) tokens
  uint32_t* __restrict__ ukeys = bkeys + (size_t)u * kstride;
  const float* __restrict__ sg = sigma + (size_t)u * cap;
  const int span = bs > 256 ? bs : 256;
  const int sp_lo = sl * (kBlkSpan / span);
  const int sp_hi = min((n + span - 1) / span, sp_lo + kBlkSpan / span);
  const int G = (bs < 256 ? bs : 256) / 4;  // lanes per block in one load
  for (int s0 = sp_lo + wv; s0 < sp_hi; s0 += kBlkBatch * kWaves) {
    float m[kBlkBatch];
#pragma unroll
    for (int i = 0; i < kBlkBatch; ++i) m[i] = -INFINITY;
    for (int c = 0; c < span; c += 256) {
      float4 x[kBlkBatch];
#pragma unroll
      for (int i = 0; i < kBlkBatch; ++i) {  // clamped: every load unconditional and inside the unit's row
        const int t = (s0 + i * kWaves) * span + c + 4 * lane;
        x[i] = *reinterpret_cast<const float4*>(sg + min(t, cap - 4));
      }
#pragma unroll
      for (int i = 0; i < kBlkBatch; ++i) {
        const int t = (s0 + i * kWaves) * span + c + 4 * lane;
        const bool in = s0 + i * kWaves < sp_hi;
        const float a = fmaxf(in && t < n ? x[i].x : -INFINITY, in && t + 1 < n ? x[i].y : -INFINITY);
        const float b = fmaxf(in && t + 2 < n ? x[i].z : -INFINITY, in && t + 3 < n ? x[i].w : -INFINITY);
        m[i] = fmaxf(m[i], fmaxf(a, b));
      }
    }
#pragma unroll
    for (int i = 0; i < kBlkBatch; ++i) {
      for (int off = 1; off < G; off <<= 1) m[i] = fmaxf(m[i], __shfl_xor(m[i], off));
      const int j = ((s0 + i * kWaves) * span + 4 * lane) >> lgb;
      if ((lane & (G - 1)) == 0 && s0 + i * kWaves < sp_hi && j < nblk) st_dev32(&ukeys[j], float_key(m[i]));
    }
  }

  // ---- arrival; the unit's last workgroup selects --------------------------------
  if (!arrive_is_last(&counter[u], gridDim.x, &s_last)) return;
  for (int j = tid; j < nblk; j += kThreads) s_bkey[j] = ld_dev32(&ukeys[j]);
  __syncthreads();

  // the kb best blocks: entry j = i*kThreads + tid
  uint64_t c[kBlkPer];  // 0: no block
#pragma unroll
  for (int i = 0; i < kBlkPer; ++i) {
    const int j = i * kThreads + tid;
    c[i] = (j < nblk) ? (((uint64_t)s_bkey[j] << 32) | (uint64_t)(~(uint32_t)j)) : 0ull;
  }
  auto get = [&](int j) { return ((uint64_t)s_bkey[j] << 32) | (uint64_t)(~(uint32_t)j); };
  auto fill = [] {};  // the keys are in LDS already
  const uint64_t T = hist_select<kThreads>(c, nblk, kb, get, fill, s_hist, s_wsum, s_res, s_mm, s_small);
  bool sel[kBlkPer];
#pragma unroll
  for (int i = 0; i < kBlkPer; ++i) sel[i] = c[i] && c[i] >= T;
  int at[kBlkPer];
  ordered_positions<kBlkPer, kWaves>(sel, at, s_wsum, reinterpret_cast<int*>(s_hist));
  // (every read of s_bkey is behind the barriers of ordered_positions)
#pragma unroll
  for (int i = 0; i < kBlkPer; ++i)
    if (sel[i]) s_bkey[at[i]] = (uint32_t)(i * kThreads + tid);
  __syncthreads();
  for (int i = tid; i < row; i += kThreads) {
    const int t = (int)s_bkey[i >> lgb] * bs + (i & (bs - 1));  // i >> lgb < kb = nb here
    out[i] = (t < n) ? t : -1;
  }
  if (tid == 0) counter[u] = 0u;  // ready for the next call on this workspace
}

}  // namespace

hipError_t launch_topk_blocks(const bkv_layout& L, const float* sigma, const SeqArg& len, int max_len, int nb,
                              int lgb, int32_t* idx, uint32_t* bkeys, int kstride, uint32_t* counter, hipStream_t s) {
  const int units = L.batch * L.n_kv_heads;
  const int ns = (max_len + kBlkSpan - 1) / kBlkSpan;
  (void)hipGetLastError();  // report only this call's launch
  topk_blocks_kernel<<<dim3(ns > 0 ? ns : 1, units), kThreads, 0, s>>>(sigma, idx, len, L.n_kv_heads, L.capacity, nb,
                                                                       lgb, bkeys, kstride, counter);
  return hipGetLastError();
}

hipError_t launch_topk(const bkv_layout& L, const float* sigma, const SeqArg& len, int max_len, int k, int W,
                       int32_t* idx, uint64_t* cand, uint32_t* counter, hipStream_t s) {
  const int units = L.batch * L.n_kv_heads;
  const int max_sel = max_len > W ? max_len - W : 0;  // the longest range selected from
  const int S = topk_slice(units, max_sel, k);
  (void)hipGetLastError();  // report only this call's launches
  if (S == 0) {
    topk_kernel<<<units, kThreads, 0, s>>>(sigma, idx, len, L.n_kv_heads, L.capacity, k, W);
  } else {
    const int ns = (max_sel + S - 1) / S;
    const int slots = ns * k;
    const dim3 grid(ns > 0 ? ns : 1, units);
    if ((size_t)slots * 8 <= (size_t)kLocalMax * 4) {  // the merge fits the slice stage's LDS: fused
      topk_slices_kernel<true><<<grid, kLocalThreads, 0, s>>>(sigma, cand, counter, idx, len, L.n_kv_heads,
                                                              L.capacity, k, W, S, slots);
    } else {
      topk_slices_kernel<false><<<grid, kLocalThreads, 0, s>>>(sigma, cand, counter, idx, len, L.n_kv_heads,
                                                               L.capacity, k, W, S, slots);
      topk_merge_kernel<<<units, kThreads, 0, s>>>(cand, idx, len, L.n_kv_heads, k, W, S, slots);
    }
  }
  return hipGetLastError();
}

}  // namespace bkv
