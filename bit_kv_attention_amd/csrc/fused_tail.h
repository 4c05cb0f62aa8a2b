// fused_tail.h -- the end of the fused decode step (qattn_decode_fused): what
// follows the approximate scan inside the same launch, in each of a unit's
// nsplit workgroups (one split each), so that the selection and the exact
// correction need no launch of their own (JetFire README, introduction:
// approximate attention, top-k selection, high-precision correction of the
// selected tokens).  Written for latency: each step costs a round trip to
// the device's coherence point, and there are four of them after the scan.
//
//  1. Publish.  During the scan every workgroup histogrammed its split's
//     selection scores by the top kFBinBits bits of their order-preserving
//     keys (monotone in the score, no range needed).  It finds the bin D_s
//     of its own kk-th largest score, lists its entries of bins >= D_s in
//     index order (composites) in the workspace with the list's size and
//     D_s, and meets the unit's other workgroups at a barrier.
//  2. Threshold.  Each loads every list into LDS.  A split's kk-th largest
//     score is never above the unit's, so the bin D of the unit's kk-th
//     largest is >= Dmax = max D_s, and in the bins >= Dmax the lists hold
//     every entry of the unit: their histogram there is the unit's.  It gives
//     D and how many of D's entries are taken; those are ranked exactly and
//     T = the needD-th largest.  The selected set {t : composite(t) >= T} is
//     the set topk_select finds.  (Lists too long for LDS -- many equal
//     scores -- take a radix select over the lists in the workspace.)
//  3. Correction.  The split's own selected tokens in passes of kFPass:
//     exact logits from the fp16 shadow rows, approximate logits recomputed
//     from the codes (correct_lane.h), the exact state online over the
//     passes, the approximate terms relative to the split's maximum; the
//     split state then loses the selected tokens' approximate terms and gains
//     their exact ones (the formula of correct.hip, per split).  A split
//     whose every token is selected keeps only the exact state.
//  4. Output.  The corrected split record goes to the workspace; the unit's
//     last workgroup to arrive merges the records into the output, writes
//     the unit's row of idx from the lists, and zeroes the counters for the
//     next call.
// Everything one workgroup hands to another goes through agent-scope atomic
// accesses and the counters of select_lds.h.
#pragma once

#include "bkv_internal.h"
#include "correct_lane.h"
#include "select_lds.h"

namespace bkv {

__device__ inline uint32_t fbin(float s) { return float_key(s) >> (32 - kFBinBits); }
__device__ inline uint32_t fbin_c(uint64_t c) { return (uint32_t)(c >> (64 - kFBinBits)); }

// Sum over the 64 lanes of a wave, in every lane.
__device__ inline float wave_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Ordered compaction over entries [0, n) by the NW waves of the workgroup:
// wave w walks the contiguous range [w*R, w*R + R) (R a multiple of 64) in
// steps of 64, counts the entries with pred(i) by ballots, the wave counts
// are prefix-summed through LDS, and a second walk calls emit(position, i)
// for each in index order.  Returns the count (every thread).  s_wc: NW ints.
template <int NW, typename Pred, typename Emit>
__device__ inline int ordered_compact(int n, Pred pred, Emit emit, int* s_wc) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
  const int R = ((n + NW * 64 - 1) / (NW * 64)) * 64;
  const int lo = wv * R, hi = min(n, lo + R);
  int cnt = 0;
  for (int b = lo; b < hi; b += 64) {
    const int i = b + lane;
    cnt += __popcll(__ballot(i < hi && pred(i)));
  }
  __syncthreads();  // (s_wc may still be read by a previous call)
  if (lane == 0) s_wc[wv] = cnt;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = s_wc[w];
    base += (w < wv) ? c : 0;
    total += c;
  }
  const uint64_t below = (1ull << lane) - 1;
  for (int b = lo; b < hi; b += 64) {
    const int i = b + lane;
    const bool p = i < hi && pred(i);
    const uint64_t m = __ballot(p);
    if (p) emit(base + __popcll(m & below), i);
    base += __popcll(m);
  }
  return total;
}

// Everything the tail needs from the scan kernel.
template <int G>
struct FusedCtx {
  int tid, u, b, kvh, split, len, t_begin, t_end, nsplit, chunk, ksel, cap, mshift, Hq;
  uint32_t top_bin;  // the highest bin of the split's scores (0 when empty)
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint32_t* kmeta;
  const uint32_t* vmeta;
  const uint16_t* ksh;  // the unit's shadow rows
  const uint16_t* vsh;
  float* pm;
  float* pl;
  float* pacc;
  int32_t* idx;
  FusedArgs fa;
  // LDS of the scan, reused
  const uint16_t (*s_q)[kHeadDim];
  float* s_split;   // the split's selection scores (kSelStage floats); then the unit's lists
  uint32_t* s_fh;   // the split's histogram (kFBins words); then bin D's entries, the own tokens
  float* s_acc;     // kScanWaves * G * kHeadDim floats: select scratch, correction partials
  float* s_lg;      // >= 2 * kFPass * G floats
  float* s_w;       // >= 2 * kFPass * G floats
};

constexpr int kFUnion = kSelStage / 2;  // list entries (composites) the LDS takes: the scores' room
constexpr int kFBinD = kFBins / 2;      // bin-D entries the LDS takes: the histogram's room
constexpr int kFWin = 512;              // bins of the window histogram above Dmax
constexpr int kFStage = 512;            // list entries a wave stages in LDS (the correction partials' room)

// rm, rl, ra: this thread's (head, channel) pairs e = tid + 512 r of the
// split's approximate state (max in log2 units, denominator, value sum).
template <int KB, int VB, int G>
__device__ __forceinline__ void fused_tail(const FusedCtx<G>& x, const float (&rm)[G / 4],
                                           const float (&rl)[G / 4], const float (&ra)[G / 4]) {
  constexpr int NTH = 64 * kScanWaves;
  constexpr int NW = kScanWaves;
  constexpr int NR = G * kHeadDim / NTH;
  constexpr float kLog2eF = 1.4426950408889634f;
  const int tid = x.tid, lane = tid & 63, wv = tid >> 6;
  const int kk = min(x.ksel, x.len);
  const int len_s = max(0, x.t_end - x.t_begin);
  const bool partial = 0 < kk && kk < x.len;  // (the same in the unit's workgroups)
  uint32_t* ctr = x.fa.ctr + 2 * (size_t)x.u;
  uint64_t* lists = x.fa.dlist + (size_t)x.u * x.nsplit * x.chunk;  // split s at s * chunk
  uint32_t* cnts = x.fa.dcnt + (size_t)x.u * x.nsplit;  // list sizes
  uint32_t* dsv = x.fa.dsv + (size_t)x.u * x.nsplit;    // the splits' D_s
  uint64_t* s_union = reinterpret_cast<uint64_t*>(x.s_split);
  uint64_t* s_dl = reinterpret_cast<uint64_t*>(x.s_fh);
  uint32_t* s_sel = x.s_fh;  // the split's own selected tokens (offsets), once the threshold is known
  __shared__ int s_res[8];
  __shared__ int s_wsum[NW];
  __shared__ float s_mm[2 * NW];
  __shared__ uint64_t s_small[65];
  __shared__ uint64_t s_T;
  __shared__ int s_dc[kFMaxSplits + 1];  // list offsets (prefix sums of the sizes)
  __shared__ int s_flag;
  __shared__ int s_n;
  __shared__ uint32_t s_dmax;

  int n_sel = 0;   // own selected tokens in s_sel
  uint64_t T = 0;  // partial: the threshold composite
  bool in_lds = false;
  int32_t* row = x.idx + (size_t)x.u * x.ksel;  // the unit's row of idx
  const uint64_t below = (1ull << lane) - 1;
  if (partial) {
    // ---- 1. publish ------------------------------------------------------------------
    const int kks = min(kk, len_s);
    uint32_t Ds = 0;  // (a split with at most kk tokens lists them all)
    if (kks < len_s) {
      // the bin of the split's kks-th largest: wave 0 walks down from the
      // split's top bin, 64 bins at a time (lane l takes bin top - l)
      if (wv == 0) {
        int acc = 0;
        for (int top = (int)x.top_bin; top >= 0; top -= 64) {
          const int b = top - lane;
          const int inc = wave_incl_scan((b >= 0) ? (int)x.s_fh[b] : 0);
          const uint64_t hit = __ballot(acc + inc >= kks);
          if (hit) {
            if (lane == __builtin_ctzll(hit)) s_res[0] = b;
            break;
          }
          acc += __shfl(inc, 63);
        }
      }
      __syncthreads();
      Ds = (uint32_t)s_res[0];
    }
    // the split's entries of bins >= Ds in index order: each wave stages the
    // offsets of its contiguous range in LDS in one pass, then copies them
    // out behind the lower waves' (a wave with more than kFStage of them --
    // many equal scores -- sends the workgroup to the two-pass compaction)
    uint64_t* mylist = lists + (size_t)x.split * x.chunk;
    int nlist = 0;
    {
      uint32_t* stage = reinterpret_cast<uint32_t*>(x.s_acc) + wv * kFStage;
      // wave range: a multiple of 256 entries (lane l reads entries 4l..4l+3
      // of each 256 with one 16-byte LDS read; the reads stay inside the
      // kSelStage scores)
      const int R = ((len_s + NW * 256 - 1) / (NW * 256)) * 256;
      const int lo = wv * R, hi = min(len_s, lo + R);
      int cnt = 0;
      for (int b0 = lo; b0 < hi; b0 += 512) {
        floatx4 v[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) v[r] = *reinterpret_cast<const floatx4*>(&x.s_split[b0 + 256 * r + 4 * lane]);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int i0 = b0 + 256 * r + 4 * lane;
          bool p[4];
          int c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = i0 + j < hi && fbin(v[r][j]) >= Ds;
            c += p[j] ? 1 : 0;
          }
          const int inc = wave_incl_scan(c);
          int q = cnt + inc - c;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (p[j]) {
              if (q < kFStage) stage[q] = (uint32_t)(i0 + j);
              ++q;
            }
          }
          cnt += __shfl(inc, 63);
        }
      }
      if (lane == 0) s_wsum[wv] = cnt;
      __syncthreads();
      int base = 0;
      bool ovf = false;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = s_wsum[w];
        base += (w < wv) ? c : 0;
        nlist += c;
        ovf = ovf || c > kFStage;
      }
      if (!ovf) {
        for (int j = lane; j < cnt; j += 64) {
          const int i = (int)stage[j];
          st_dev64(&mylist[base + j], composite(x.s_split[i], x.t_begin + i));
        }
      } else {
        ordered_compact<NW>(
            len_s, [&](int i) { return fbin(x.s_split[i]) >= Ds; },
            [&](int q, int i) { st_dev64(&mylist[q], composite(x.s_split[i], x.t_begin + i)); }, s_wsum);
      }
    }
    if (tid == 0) {
      st_dev32(&cnts[x.split], (uint32_t)nlist);
      st_dev32(&dsv[x.split], Ds);
      s_dmax = 0u;  // (ordered before its updates below by the barrier)
    }
    unit_barrier(&ctr[0], (uint32_t)x.nsplit, x.fa.flag);

    // ---- 2. threshold ---------------------------------------------------------------
    {  // list sizes (prefix sums) and Dmax
      const int q = min(tid, x.nsplit - 1);  // (unconditional loads: a branch around a load waits for it)
      const int c = (int)ld_dev32(&cnts[q]);
      const uint32_t d = ld_dev32(&dsv[q]);
      if (tid < x.nsplit) {
        s_dc[tid + 1] = c;
        atomicMax(&s_dmax, d);
      }
      __syncthreads();
      if (tid == 0) {
        s_dc[0] = 0;
        for (int s = 0; s < x.nsplit; ++s) s_dc[s + 1] += s_dc[s];
        s_n = 0;
      }
      __syncthreads();
    }
    const uint32_t Dmax = s_dmax;
    const int total = s_dc[x.nsplit];
    in_lds = total <= kFUnion;
    if (in_lds) {
      // the lists to LDS: wave w loads the lists of splits w, w + NW, ..., 8
      // unconditional loads per lane in flight together
      for (int i = tid; i < kFWin; i += NTH) x.s_fh[i] = 0u;
      for (int s = wv; s < x.nsplit; s += NW) {
        const int o = s_dc[s], c = s_dc[s + 1] - o;
        const uint64_t* src = lists + (size_t)s * x.chunk;
        constexpr int kBat = 8;
        for (int p0 = 0; p0 < c; p0 += 64 * kBat) {
          uint64_t v[kBat];
#pragma unroll
          for (int r = 0; r < kBat; ++r) v[r] = ld_dev64(&src[min(p0 + 64 * r + lane, c - 1)]);
#pragma unroll
          for (int r = 0; r < kBat; ++r) {
            const int p = p0 + 64 * r + lane;
            if (p < c) s_union[o + p] = v[r];
          }
        }
      }
      __syncthreads();
      // their histogram in the bins Dmax .. Dmax + kFWin - 2 (the unit's
      // there; the last counter takes every bin above), then D: thread tid
      // owns counter kFWin - 1 - tid
      for (int i = tid; i < total; i += NTH) {
        const uint32_t b = fbin_c(s_union[i]);
        if (b >= Dmax) atomicAdd(&x.s_fh[min(b - Dmax, (uint32_t)kFWin - 1)], 1u);
      }
      __syncthreads();
      {
        const int mine = (tid < kFWin) ? (int)x.s_fh[kFWin - 1 - tid] : 0;
        int tot;
        const int above = block_excl_scan<NW>(mine, s_wsum, tot);
        if (above < kk && above + mine >= kk) {
          s_res[0] = (int)Dmax + kFWin - 1 - tid;
          s_res[1] = above;
          s_res[2] = mine;
          s_res[3] = (tid == 0);  // the top counter: bins merged
        }
        __syncthreads();  // (every read of the counters is done: their room takes bin D's entries)
      }
      if (s_res[3]) {  // the kk-th largest lies kFWin - 1 or more bins above Dmax: the full histogram
        for (int i = tid; i < kFBins; i += NTH) x.s_fh[i] = 0u;
        __syncthreads();
        for (int i = tid; i < total; i += NTH) {
          const uint32_t b = fbin_c(s_union[i]);
          if (b >= Dmax) atomicAdd(&x.s_fh[b], 1u);
        }
        __syncthreads();
        constexpr int PB = kFBins / NTH;
        int mine = 0;
#pragma unroll
        for (int i = 0; i < PB; ++i) mine += (int)x.s_fh[kFBins - 1 - PB * tid - i];
        int tot;
        int above = block_excl_scan<NW>(mine, s_wsum, tot);
        if (above < kk && above + mine >= kk) {
          for (int i = 0; i < PB; ++i) {
            const int h = (int)x.s_fh[kFBins - 1 - PB * tid - i];
            if (above + h >= kk) {
              s_res[0] = kFBins - 1 - PB * tid - i;
              s_res[1] = above;
              s_res[2] = h;
              break;
            }
            above += h;
          }
        }
        __syncthreads();
      }
      const uint32_t D = (uint32_t)s_res[0];
      const int needD = kk - s_res[1], inD = s_res[2];
      if (needD == inD) {  // all of bin D
        if (tid == 0) s_T = (uint64_t)D << (64 - kFBinBits);
      } else if (inD <= kFBinD) {
        for (int i = tid; i < total; i += NTH) {
          const uint64_t e = s_union[i];
          if (fbin_c(e) == D) s_dl[atomicAdd(&s_n, 1)] = e;
        }
        __syncthreads();
        const int m = inD;
        if (m <= NTH) {  // rank every entry against all (distinct composites), 8 reads in flight
          if (tid < m) {
            const uint64_t c = s_dl[tid];
            int r = 0, j = 0;
            for (; j + 8 <= m; j += 8) {
#pragma unroll
              for (int z = 0; z < 8; ++z) r += (s_dl[j + z] > c) ? 1 : 0;
            }
            for (; j < m; ++j) r += (s_dl[j] > c) ? 1 : 0;
            if (r == needD - 1) s_T = c;
          }
        } else {
          constexpr int PER = kFBinD / NTH;
          uint64_t c[PER];
#pragma unroll
          for (int j = 0; j < PER; ++j) c[j] = (j * NTH + tid < m) ? s_dl[j * NTH + tid] : 0ull;
          auto get = [&](int i) { return s_dl[i]; };
          auto fill = [] {};  // (the entries are in LDS already)
          const uint64_t t = hist_select<NTH>(c, m, needD, get, fill, reinterpret_cast<uint32_t*>(x.s_acc),
                                              s_wsum, s_res, s_mm, s_small);
          if (tid == 0) s_T = t;
        }
      } else {  // a crowded bin D: radix select among its entries in LDS
        auto get = [&](int i) -> uint64_t {
          const uint64_t e = s_union[i];
          return fbin_c(e) == D ? e : 0ull;
        };
        const uint64_t t = lds_threshold<NTH>(get, total, needD, reinterpret_cast<uint32_t*>(x.s_acc), s_wsum, s_res);
        if (tid == 0) s_T = t;
      }
    } else {  // many equal scores: a radix select over the lists in the workspace (bins >= Dmax)
      auto get = [&](int i) -> uint64_t {
        const int s = i / x.chunk, p = i - s * x.chunk;
        if (p >= s_dc[s + 1] - s_dc[s]) return 0ull;
        const uint64_t c = ld_dev64(&lists[i]);
        return fbin_c(c) >= Dmax ? c : 0ull;
      };
      const uint64_t t = lds_threshold<NTH>(get, x.nsplit * x.chunk, kk, reinterpret_cast<uint32_t*>(x.s_acc),
                                            s_wsum, s_res);
      if (tid == 0) s_T = t;
    }
    __syncthreads();
    T = s_T;
    // the split's own selected tokens
    if (in_lds) {  // in index order, straight into their place in the row of idx
      const int o = s_dc[x.split], c = s_dc[x.split + 1] - o;
      int before = 0;  // selected tokens of the lower splits
      for (int i = tid; i < o; i += NTH) before += (s_union[i] >= T) ? 1 : 0;
      int tot;
      (void)block_excl_scan<NW>(before, s_wsum, tot);
      before = tot;
      n_sel = ordered_compact<NW>(
          c, [&](int i) { return s_union[o + i] >= T; },
          [&](int q, int i) {
            const int t = (int)~(uint32_t)(s_union[o + i] & 0xFFFFFFFFu);
            s_sel[q] = (uint32_t)(t - x.t_begin);
            if (before + q < x.ksel) row[before + q] = t;
          },
          s_wsum);
      if (x.split == 0)
        for (int j = kk + tid; j < x.ksel; j += NTH) row[j] = -1;
    } else {  // (any order; the unit's last workgroup writes idx from the lists)
      if (tid == 0) s_n = 0;
      __syncthreads();
      for (int i = tid; i < len_s; i += NTH)
        if (composite(x.s_split[i], x.t_begin + i) >= T) s_sel[atomicAdd(&s_n, 1)] = (uint32_t)i;
      __syncthreads();
      n_sel = s_n;
    }
    __syncthreads();
    n_sel = min(n_sel, x.ksel);  // (<= min(kk, len_s); the clamp only guards the lists)
  } else {
    if (kk > 0) {  // every token is selected
      for (int i = tid; i < len_s; i += NTH) {
        s_sel[i] = (uint32_t)i;
        row[x.t_begin + i] = x.t_begin + i;
      }
      n_sel = len_s;
    }
    if (x.split == 0)
      for (int j = kk + tid; j < x.ksel; j += NTH) row[j] = -1;
    __syncthreads();
  }

  // ---- 3. correction of this split's state ------------------------------------------
  float ex_m[NR], ex_l[NR], ex_a[NR], ap_l[NR], ap_a[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    ex_m[r] = -INFINITY;
    ex_l[r] = ex_a[r] = ap_l[r] = ap_a[r] = 0.f;
  }
  if (n_sel > 0) {
    const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2eF;
    __shared__ float s_qrun[G][kHeadDim / 16];  // sums of 16-channel runs of the query rows
    __shared__ float s_rmh[G];                   // the split's approximate maximum per head
    __shared__ int s_tok[kFPass];
    __shared__ float s_mx[G];
    __shared__ float s_ls[2][G];
    if (tid < G * (kHeadDim / 16)) {
      const int h = tid / (kHeadDim / 16), p = tid % (kHeadDim / 16);
      float r = 0.f;
      for (int c = 0; c < 16; ++c) r += h2f(x.s_q[h][16 * p + c]);
      s_qrun[h][p] = r;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int e = tid + NTH * r;
      if ((e & (kHeadDim - 1)) == 0) s_rmh[e / kHeadDim] = rm[r];
    }
    const uint4(*qh)[kHeadDim / 8] = reinterpret_cast<const uint4(*)[kHeadDim / 8]>(&x.s_q[0][0]);
    float(*s_lg)[kFPass][G] = reinterpret_cast<float(*)[kFPass][G]>(x.s_lg);
    float(*s_w)[kFPass][G] = reinterpret_cast<float(*)[kFPass][G]>(x.s_w);
    float(*s_part)[4][G][kHeadDim] = reinterpret_cast<float(*)[4][G][kHeadDim]>(x.s_acc);
    const int tl = tid >> 3, part = tid & 7;             // logits: 8 threads per token
    const int c = tid & (kHeadDim - 1), qtr = tid >> 7;  // values: (channel, quarter of the pass)
    for (int p0 = 0; p0 < n_sel; p0 += kFPass) {
      const int np = min(kFPass, n_sel - p0);
      if (tid < kFPass) s_tok[tid] = (tid < np) ? x.t_begin + (int)s_sel[p0 + tid] : -1;
      __syncthreads();
      // loads: every one unconditional (an empty slot reads token 0, present
      // whenever a token is selected) and in flight before the first is used
      const int tsel = s_tok[tl];
      KeyRun<KB, true, true> kr;
      kr.load(x.ksh, x.kbase, x.kmeta, x.cap, max(tsel, 0), part, x.mshift);
      constexpr int kQ = kFPass / 4;
      uint16_t vx16[kQ];
      ValueCode<VB> vcd[kQ];
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const int t = max(s_tok[qtr * kQ + j], 0);
        vcd[j].load(x.vbase, x.vmeta, x.cap, t, c, x.mshift);
        vx16[j] = x.vsh[(size_t)t * kHeadDim + c];
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        float ex[G], ap[G];
        run_logits<KB, G, true, true, false, 0>(kr, part, qh, s_qrun, nullptr, nullptr, nullptr, ex, ap);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          ex[h] = sum8(ex[h]);
          ap[h] = sum8(ap[h]);
        }
        if (part == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            s_lg[0][tl][h] = (tsel >= 0) ? ex[h] * sm2 : -INFINITY;
            s_lg[1][tl][h] = (tsel >= 0) ? ap[h] * sm2 : -INFINITY;
          }
        }
      }
      __syncthreads();
      // per (exact/approximate, head): lane t of a wave takes token t -- the
      // weights (exact: relative to the pass maximum; approximate: to the
      // split's), their sum and the pass maximum by wave reductions
      for (int cb = wv; cb < 2 * G; cb += NW) {
        const int ty = cb / G, h = cb % G;
        const bool ok = s_tok[lane] >= 0;
        const float lg = s_lg[ty][lane][h];
        const float ref = (ty == 0) ? wave_minmax<true>(lg) : s_rmh[h];
        const float wgt = ok ? __builtin_amdgcn_exp2f(lg - ref) : 0.f;
        s_w[ty][lane][h] = wgt;
        const float l = wave_sum(wgt);
        if (lane == 0) {
          s_ls[ty][h] = l;
          if (ty == 0) s_mx[h] = ref;
        }
      }
      __syncthreads();
      {
        float ea[G], aa[G];
#pragma unroll
        for (int h = 0; h < G; ++h) ea[h] = aa[h] = 0.f;
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
          const int t2 = qtr * kQ + j;
          const float vx = h2f(vx16[j]);
          const float vq = vcd[j].value(max(s_tok[t2], 0), c);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            ea[h] = fmaf(s_w[0][t2][h], vx, ea[h]);
            aa[h] = fmaf(s_w[1][t2][h], vq, aa[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s_part[0][qtr][h][c] = ea[h];
          s_part[1][qtr][h][c] = aa[h];
        }
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int e = tid + NTH * r, hh = e / kHeadDim, cc = e & (kHeadDim - 1);
        const float pe = s_part[0][0][hh][cc] + s_part[0][1][hh][cc] + s_part[0][2][hh][cc] + s_part[0][3][hh][cc];
        const float pa = s_part[1][0][hh][cc] + s_part[1][1][hh][cc] + s_part[1][2][hh][cc] + s_part[1][3][hh][cc];
        const float mp = s_mx[hh];  // finite: the pass has a token
        const float mn = fmaxf(ex_m[r], mp);
        const float f0 = __builtin_amdgcn_exp2f(ex_m[r] - mn), f1 = __builtin_amdgcn_exp2f(mp - mn);
        ex_a[r] = fmaf(ex_a[r], f0, pe * f1);
        ex_l[r] = fmaf(ex_l[r], f0, s_ls[0][hh] * f1);
        ex_m[r] = mn;
        ap_a[r] += pa;
        ap_l[r] += s_ls[1][hh];
      }
    }
  }

  // ---- 4. the corrected record; the unit's last workgroup writes the output ----------
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = tid + NTH * r, hh = e / kHeadDim, cc = e & (kHeadDim - 1);
    float M = rm[r], l = rl[r], a = ra[r];
    if (n_sel > 0) {
      if (n_sel == len_s) {  // every token of the split is selected
        M = ex_m[r];
        l = ex_l[r];
        a = ex_a[r];
      } else {
        const float Mp = fmaxf(M, ex_m[r]);
        const float fa = __builtin_amdgcn_exp2f(M - Mp), fe = __builtin_amdgcn_exp2f(ex_m[r] - Mp);
        l = fmaf(fa, fmaxf(l - ap_l[r], 0.f), fe * ex_l[r]);
        a = fmaf(fa, a - ap_a[r], fe * ex_a[r]);
        M = Mp;
      }
    }
    const size_t rec = ((size_t)x.b * x.Hq + (size_t)x.kvh * G + hh) * x.nsplit + x.split;
    st_devf(&x.pacc[rec * kHeadDim + cc], a);
    if (cc == 0) {
      st_devf(&x.pm[rec], M);
      st_devf(&x.pl[rec], l);
    }
  }
  if (!arrive_is_last(&ctr[1], (uint32_t)x.nsplit, &s_flag)) return;

  // the records, in batches of kB (their loads all in flight together)
  constexpr int kB = 16;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = tid + NTH * r, hh = e / kHeadDim, cc = e & (kHeadDim - 1);
    const size_t rec0 = ((size_t)x.b * x.Hq + (size_t)x.kvh * G + hh) * x.nsplit;
    float m = -INFINITY, l = 0.f, a = 0.f;
    for (int s0 = 0; s0 < x.nsplit; s0 += kB) {
      float ms[kB], ls[kB], as[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const size_t s = (size_t)min(s0 + j, x.nsplit - 1);
        ms[j] = ld_devf(&x.pm[rec0 + s]);
        ls[j] = ld_devf(&x.pl[rec0 + s]);
        as[j] = ld_devf(&x.pacc[(rec0 + s) * kHeadDim + cc]);
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (s0 + j < x.nsplit) {
          const float mn = fmaxf(m, ms[j]);
          const float ref = (mn == -INFINITY) ? 0.f : mn;
          const float f0 = __builtin_amdgcn_exp2f(m - ref), f1 = __builtin_amdgcn_exp2f(ms[j] - ref);
          a = fmaf(a, f0, as[j] * f1);
          l = fmaf(l, f0, ls[j] * f1);
          m = mn;
        }
      }
    }
    x.fa.out[(rec0 / x.nsplit) * kHeadDim + cc] = (x.len > 0) ? a / l : 0.f;
  }
  if (partial && !in_lds) {  // the row of idx: the listed composites >= T, in list order = token order
    auto get = [&](int i) -> uint64_t {
      const int s = i / x.chunk, p = i - s * x.chunk;
      return (p < s_dc[s + 1] - s_dc[s]) ? ld_dev64(&lists[i]) : 0ull;
    };
    const int n = ordered_compact<NW>(
        x.nsplit * x.chunk, [&](int i) { return get(i) >= T; },
        [&](int q, int i) {
          if (q < x.ksel) row[q] = (int32_t)~(uint32_t)(get(i) & 0xFFFFFFFFu);
        },
        s_wsum);
    for (int j = n + tid; j < x.ksel; j += NTH) row[j] = -1;
  }
  if (tid == 0) {
    ctr[0] = 0u;
    ctr[1] = 0u;
  }
}

}  // namespace bkv
