// fused_tail.h -- the end of the fused decode step (qattn_decode_fused): what
// follows the approximate scan inside the same launch, in each of a unit's
// nsplit workgroups (one split each), so that the selection and the exact
// correction need no launch of their own (JetFire README, introduction:
// approximate attention, top-k selection, high-precision correction of the
// selected tokens).
//
//  1. Threshold.  During the scan every workgroup histogrammed its split's
//     selection scores by the top kFBinBits bits of their order-preserving
//     keys (bins are monotone in the score and need no range).  It adds its
//     histogram into the unit's (global atomics on the non-empty bins) and
//     meets the unit's other workgroups at a barrier.  Each then reads the
//     unit's histogram and finds the bin D that holds the kk-th largest score
//     and how many of D's entries are taken (needD).  If that is all of D the
//     threshold is D's lowest composite.  Otherwise every workgroup lists its
//     split's entries of bin D (composites) in the workspace, they meet again,
//     and each ranks the unit's bin-D entries exactly: T = the needD-th
//     largest of them (in LDS when they fit kFDList, else by a radix select
//     over the lists in the workspace).  The selected set is
//     {t : composite(t) >= T}, the same set topk_select finds.
//  2. Own tokens.  Each workgroup takes the selected tokens of its own split
//     (from the scores it still holds in LDS), in index order, into its list
//     slot in the workspace and into LDS.
//  3. Correction.  Passes of kFPass tokens: exact logits from the fp16 shadow
//     rows, approximate logits recomputed from the codes (correct_lane.h),
//     exact state online over the passes, approximate terms relative to the
//     split's own maximum; then the split state loses the selected tokens'
//     approximate terms and gains their exact ones (the formula of
//     correct.hip, per split).  A split whose every token is selected keeps
//     only the exact state.
//  4. Output.  The corrected split record goes to the workspace; the unit's
//     last workgroup to arrive merges the nsplit records into the output,
//     writes the unit's row of idx from the per-split lists, and zeroes the
//     histogram and the counters for the next call.
// Everything one workgroup hands to another goes through agent-scope atomic
// accesses and the counters of select_lds.h.
#pragma once

#include "bkv_internal.h"
#include "correct_lane.h"
#include "select_lds.h"

namespace bkv {

__device__ inline uint32_t fbin(float s) { return float_key(s) >> (32 - kFBinBits); }

// Everything the tail needs from the scan kernel.
template <int G>
struct FusedCtx {
  int tid, u, b, kvh, split, len, t_begin, t_end, nsplit, chunk, ksel, cap, mshift, Hq;
  const uint8_t* kbase;
  const uint8_t* vbase;
  const uint32_t* kmeta;
  const uint32_t* vmeta;
  const uint16_t* ksh;  // the unit's shadow rows
  const uint16_t* vsh;
  float* pm;
  float* pl;
  float* pacc;
  uint64_t* tkc;        // per-split lists of selected tokens: [U][nsplit][ksel]
  int32_t* idx;
  FusedArgs fa;
  // LDS of the scan, reused
  const uint16_t (*s_q)[kHeadDim];
  const float* s_split;  // the split's selection scores
  uint32_t* s_fh;        // the split's histogram (kFBins words); later lists
  float* s_acc;          // kScanWaves * G * kHeadDim floats
  float* s_lg;           // >= 2 * kFPass * G floats
  float* s_w;            // >= 2 * kFPass * G floats
};

// rm, rl, ra: this thread's (head, channel) pairs e = tid + 512 r of the
// split's approximate state (max in log2 units, denominator, value sum).
template <int KB, int VB, int G>
__device__ __forceinline__ void fused_tail(const FusedCtx<G>& x, const float (&rm)[G / 4],
                                                     const float (&rl)[G / 4], const float (&ra)[G / 4]) {
  constexpr int NTH = 64 * kScanWaves;
  constexpr int NR = G * kHeadDim / NTH;
  constexpr float kLog2eF = 1.4426950408889634f;
  const int tid = x.tid;
  const int kk = min(x.ksel, x.len);
  const int len_s = max(0, x.t_end - x.t_begin);
  const bool partial = 0 < kk && kk < x.len;  // (the same in the unit's workgroups)
  uint32_t* ctr = x.fa.ctr + 3 * (size_t)x.u;
  uint32_t* gh = x.fa.hist + (size_t)x.u * kFBins;
  __shared__ int s_res[8];
  __shared__ int s_wsum[kScanWaves];
  __shared__ float s_mm[2 * kScanWaves];
  __shared__ uint64_t s_small[65];
  __shared__ uint64_t s_T;
  __shared__ int s_dc[kFMaxSplits + 1];
  __shared__ int s_flag;

  // ---- 1. the threshold ---------------------------------------------------------
  uint64_t T = 0;  // every token >= T is selected (0: all of them)
  if (partial) {
    for (int i = tid; i < kFBins; i += NTH) {
      const uint32_t h = x.s_fh[i];
      if (h) atomicAdd(&gh[i], h);
    }
    unit_barrier(&ctr[0], (uint32_t)x.nsplit, x.fa.flag);
    // the bin D with  sum_{b > D} hist[b] < kk <= sum_{b >= D} hist[b]: thread
    // tid owns bins kFBins - 1 - PB*tid - i, i < PB (descending)
    constexpr int PB = kFBins / NTH;
    uint32_t hb[PB];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      hb[i] = ld_dev32(&gh[kFBins - 1 - PB * tid - i]);
      mine += (int)hb[i];
    }
    int total;
    int above = block_excl_scan<kScanWaves>(mine, s_wsum, total);
    if (above < kk && above + mine >= kk) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (above + (int)hb[i] >= kk) {
          s_res[0] = kFBins - 1 - PB * tid - i;
          s_res[1] = above;
          s_res[2] = (int)hb[i];
          break;
        }
        above += (int)hb[i];
      }
    }
    __syncthreads();
    const int D = s_res[0], needD = kk - s_res[1], inD = s_res[2];
    if (needD == inD) {  // every entry of bin D is taken
      T = (uint64_t)D << (64 - kFBinBits);
    } else {
      // this split's entries of bin D into its list (room for the whole split)
      if (tid == 0) s_res[3] = 0;
      __syncthreads();
      uint64_t* dl_u = x.fa.dlist + (size_t)x.u * x.nsplit * x.chunk;
      uint64_t* dl = dl_u + (size_t)x.split * x.chunk;
      for (int i = tid; i < len_s; i += NTH) {
        const float v = x.s_split[i];
        if (fbin(v) == (uint32_t)D) st_dev64(&dl[atomicAdd(&s_res[3], 1)], composite(v, x.t_begin + i));
      }
      __syncthreads();
      if (tid == 0) st_dev32(&x.fa.dcnt[(size_t)x.u * x.nsplit + x.split], (uint32_t)s_res[3]);
      unit_barrier(&ctr[1], (uint32_t)x.nsplit, x.fa.flag);
      if (tid < x.nsplit) s_dc[tid] = (int)ld_dev32(&x.fa.dcnt[(size_t)x.u * x.nsplit + tid]);
      __syncthreads();
      if (tid == 0) {  // list offsets
        int o = 0;
        for (int s = 0; s < x.nsplit; ++s) {
          const int c = s_dc[s];
          s_dc[s] = o;
          o += c;
        }
        s_dc[x.nsplit] = o;
      }
      __syncthreads();
      const int m = s_dc[x.nsplit];  // (== inD)
      if (m <= kFDList) {
        uint64_t* s_dl = reinterpret_cast<uint64_t*>(x.s_fh);  // (kFDList entries; the histogram is done)
        for (int s = 0; s < x.nsplit; ++s) {
          const int o = s_dc[s], c = s_dc[s + 1] - o;
          for (int p = tid; p < c; p += NTH) s_dl[o + p] = ld_dev64(&dl_u[(size_t)s * x.chunk + p]);
        }
        __syncthreads();
        if (m <= NTH) {  // rank every entry against all (distinct composites)
          if (tid < m) {
            const uint64_t v = s_dl[tid];
            int r = 0;
            for (int j = 0; j < m; ++j) r += (s_dl[j] > v) ? 1 : 0;
            if (r == needD - 1) s_T = v;
          }
        } else {
          constexpr int PER = kFDList / NTH;
          uint64_t c[PER];
#pragma unroll
          for (int j = 0; j < PER; ++j) c[j] = (j * NTH + tid < m) ? s_dl[j * NTH + tid] : 0ull;
          auto get = [&](int i) { return s_dl[i]; };
          auto fill = [] {};  // (the entries are in LDS already)
          const uint64_t t = hist_select<NTH>(c, m, needD, get, fill, reinterpret_cast<uint32_t*>(x.s_acc), s_wsum,
                                              s_res, s_mm, s_small);
          if (tid == 0) s_T = t;
        }
      } else {  // many ties of bin D: radix select over the lists in the workspace
        auto get = [&](int i) -> uint64_t {
          const int s = i / x.chunk, p = i - s * x.chunk;
          return (p < s_dc[s + 1] - s_dc[s]) ? ld_dev64(&dl_u[i]) : 0ull;
        };
        const uint64_t t = lds_threshold<NTH>(get, x.nsplit * x.chunk, needD, reinterpret_cast<uint32_t*>(x.s_acc),
                                              s_wsum, s_res);
        if (tid == 0) s_T = t;
      }
      __syncthreads();
      T = s_T;
    }
  }

  // ---- 2. this split's selected tokens, in index order ------------------------------
  constexpr int PERS = kSelStage / NTH;
  bool sel[PERS];
  int at[PERS];
#pragma unroll
  for (int j = 0; j < PERS; ++j) {
    const int i = j * NTH + tid;
    bool s = false;
    if (kk > 0 && j * NTH < len_s && i < len_s) s = !partial || composite(x.s_split[i], x.t_begin + i) >= T;
    sel[j] = s;
  }
  int n_own = 0;
  ordered_positions<PERS, kScanWaves>(sel, at, s_wsum, reinterpret_cast<int*>(x.s_lg), &n_own);
  // (at most min(kk, len_s) <= ksel; the clamp only keeps the lists in bounds
  // should a barrier ever have given up waiting)
  n_own = min(n_own, x.ksel);
  uint32_t* s_list = x.s_fh;  // (the threshold-bin entries are no longer needed)
  uint64_t* mylist = x.tkc + ((size_t)x.u * x.nsplit + x.split) * x.ksel;
#pragma unroll
  for (int j = 0; j < PERS; ++j) {
    if (sel[j] && at[j] < n_own) {
      const int i = j * NTH + tid;
      s_list[at[j]] = (uint32_t)i;
      st_dev64(&mylist[at[j]], (uint64_t)(x.t_begin + i));
    }
  }
  if (tid == 0 && x.ksel > 0) st_dev32(&x.fa.scnt[(size_t)x.u * x.nsplit + x.split], (uint32_t)n_own);

  // ---- 3. the correction of this split's state ---------------------------------------
  float ex_m[NR], ex_l[NR], ex_a[NR], ap_l[NR], ap_a[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    ex_m[r] = -INFINITY;
    ex_l[r] = ex_a[r] = ap_l[r] = ap_a[r] = 0.f;
  }
  if (n_own > 0) {
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
    const int tl = tid >> 3, part = tid & 7;          // logits: 8 threads per token
    const int c = tid & (kHeadDim - 1), qtr = tid >> 7;  // values: (channel, quarter of the pass)
    for (int p0 = 0; p0 < n_own; p0 += kFPass) {
      const int np = min(kFPass, n_own - p0);
      __syncthreads();  // (the list is complete; the previous pass is done with the LDS below)
      if (tid < kFPass) s_tok[tid] = (tid < np) ? x.t_begin + (int)s_list[p0 + tid] : -1;
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
        run_logits<KB, G, true, true, false, false>(kr, part, qh, s_qrun, nullptr, nullptr, nullptr, ex, ap);
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
      if (tid < G) {  // the pass's exact maximum per head
        float m = -INFINITY;
        for (int t2 = 0; t2 < kFPass; ++t2) m = fmaxf(m, s_lg[0][t2][tid]);
        s_mx[tid] = m;
      }
      __syncthreads();
      {  // weights: exact relative to the pass maximum, approximate to the split's
        const int h = tid & 7;
        if (h < G) {
          const bool ok = s_tok[tl] >= 0;
          s_w[0][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[0][tl][h] - s_mx[h]) : 0.f;
          s_w[1][tl][h] = ok ? __builtin_amdgcn_exp2f(s_lg[1][tl][h] - s_rmh[h]) : 0.f;
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
        if (tid < 2 * G) {
          const int ty = tid / G, h = tid % G;
          float l = 0.f;
          for (int t2 = 0; t2 < kFPass; ++t2) l += s_w[ty][t2][h];
          s_ls[ty][h] = l;
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
    if (n_own > 0) {
      if (n_own == len_s) {  // every token of the split is selected
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
  if (!arrive_is_last(&ctr[2], (uint32_t)x.nsplit, &s_flag)) return;

#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = tid + NTH * r, hh = e / kHeadDim, cc = e & (kHeadDim - 1);
    const size_t rec0 = ((size_t)x.b * x.Hq + (size_t)x.kvh * G + hh) * x.nsplit;
    float m = -INFINITY, l = 0.f, a = 0.f;
    for (int s = 0; s < x.nsplit; ++s) {
      const float ms = ld_devf(&x.pm[rec0 + s]), ls = ld_devf(&x.pl[rec0 + s]);
      const float as = ld_devf(&x.pacc[(rec0 + s) * kHeadDim + cc]);
      const float mn = fmaxf(m, ms);
      const float ref = (mn == -INFINITY) ? 0.f : mn;
      const float f0 = __builtin_amdgcn_exp2f(m - ref), f1 = __builtin_amdgcn_exp2f(ms - ref);
      a = fmaf(a, f0, as * f1);
      l = fmaf(l, f0, ls * f1);
      m = mn;
    }
    x.fa.out[(rec0 / x.nsplit) * kHeadDim + cc] = (x.len > 0) ? a / l : 0.f;
  }
  if (x.ksel > 0) {
    if (tid == 0) {
      int o = 0;
      for (int s = 0; s < x.nsplit; ++s) {
        s_dc[s] = o;
        o += (kk > 0) ? (int)ld_dev32(&x.fa.scnt[(size_t)x.u * x.nsplit + s]) : 0;
      }
      s_dc[x.nsplit] = o;
    }
    __syncthreads();
    int32_t* row = x.idx + (size_t)x.u * x.ksel;
    for (int s = 0; s < x.nsplit; ++s) {
      const int o = s_dc[s], n = s_dc[s + 1] - o;
      const uint64_t* lst = x.tkc + ((size_t)x.u * x.nsplit + s) * x.ksel;
      for (int j = tid; j < n && o + j < x.ksel; j += NTH) row[o + j] = (int32_t)ld_dev64(&lst[j]);
    }
    for (int j = s_dc[x.nsplit] + tid; j < x.ksel; j += NTH) row[j] = -1;
  }
  if (partial)
    for (int i = tid; i < kFBins; i += NTH) gh[i] = 0u;
  if (tid == 0) {
    ctr[0] = 0u;
    ctr[1] = 0u;
    ctr[2] = 0u;
  }
}

}  // namespace bkv
