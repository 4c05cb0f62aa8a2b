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
//  2. Threshold.  Each loads every list into LDS (the list sizes and the
//     first entries of every list in one round trip).  A split's kk-th
//     largest score is never above the unit's, so the bin D of the unit's
//     kk-th largest is >= Dmax = max D_s, and in the bins >= Dmax the lists
//     hold every entry of the unit: their histogram there is the unit's.  It
//     gives D and how many of D's entries are taken; those are ranked
//     exactly and T = the needD-th largest.  The selected set
//     {t : composite(t) >= T} is the set topk_select finds.  (Lists too long
//     for LDS -- many equal scores -- take a radix select over the lists in
//     the workspace.)
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
#include "quant_lane.h"
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
  // (pred is evaluated at a clamped index and combined bitwise: no branch
  // per entry)
  for (int b = lo; b < hi; b += 64) {
    const int i = b + lane;
    cnt += __popcll(__ballot((int)(i < hi) & (int)pred(min(i, hi - 1))));
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
    const bool p = (int)(i < hi) & (int)pred(min(i, hi - 1));
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
constexpr int kFSubBits = 8;            // the second level inside bin D: the next bits of the composites
constexpr int kFWin = 512;              // bins of the window histogram above Dmax
constexpr int kFStage = 512;            // list entries a wave stages in LDS (the correction partials' room)

// The loads of one correction pass of up to kFPass tokens (toks[j]; an empty
// slot, -1, reads token 0, present whenever a token is selected): thread tid
// takes the key run of token tid / 8 (channels 16 (tid % 8) ..), and lane l
// of wave w the values of channels 2l, 2l + 1 of tokens 8w .. 8w + 7 (one
// coalesced 256-byte row per token and wave).
template <int KB, int VB, int KF>
struct FPass {
  KeyRun<KB, true, true, KF> kr;
  uint32_t vx[8];     // the fp16 shadow pair
  uint32_t vd[8][2];  // the two channels' code dwords
  uint32_t vm[8];     // their group's meta word

  __device__ inline void load(const uint16_t* __restrict__ ksh, const uint8_t* __restrict__ kbase,
                              const uint32_t* __restrict__ kmeta, const uint16_t* __restrict__ vsh,
                              const uint8_t* __restrict__ vbase, const uint32_t* __restrict__ vmeta, int cap,
                              int mshift, const int* toks) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
    kr.load(ksh, kbase, kmeta, cap, max(toks[tid >> 3], 0), tid & 7, mshift);
    const int c0 = 2 * lane;
    const size_t mrow = (size_t)((c0 / kGroup) >> mshift) * cap;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = max(toks[8 * wv + j], 0);
      vx[j] = *reinterpret_cast<const uint32_t*>(vsh + (size_t)t * kHeadDim + c0);
      const uint32_t* tile = reinterpret_cast<const uint32_t*>(vbase + (size_t)(t / kTile) * v_tile_bytes(VB));
      int d0, d1, bit;
      v_code_pos(VB, t % kTile, c0, d0, bit);
      v_code_pos(VB, t % kTile, c0 + 1, d1, bit);
      vd[j][0] = tile[d0];
      vd[j][1] = tile[d1];
      vm[j] = vmeta[mrow + t];
    }
  }
  __device__ inline void zero() {
    kr.k0 = kr.k1 = (uint4){0u, 0u, 0u, 0u};
    kr.kraw[0][0] = kr.kraw[0][1] = kr.kraw[1][0] = kr.kraw[1][1] = kr.kmw = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) vx[j] = vd[j][0] = vd[j][1] = vm[j] = 0u;
  }
};

// rm, rl, ra: this thread's (head, channel) pairs e = tid + 512 r of the
// split's approximate state (max in log2 units, denominator, value sum).
// KF: the key format (0 affine keys; 1 MXFP4 keys against the fp16 query; 2
// MXFP4 keys against the MXFP4 query, whose E2M1 codes and scales the tail
// derives from the query rows by the keys' own rule, as the correction
// kernel does).
template <int KB, int VB, int G, int KF = 0>
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
  __shared__ int s_res[8];
  __shared__ int s_wsum[NW];
  __shared__ uint64_t s_T;
  __shared__ int s_dc[kFMaxSplits + 1];  // list offsets (prefix sums of the sizes)
  __shared__ int s_flag;
  __shared__ int s_n;
  __shared__ int s_more;
  __shared__ uint32_t s_junk[64];  // a lane's target for writes and counts that do not count
  __shared__ uint32_t s_dmax;

  int n_sel = 0;   // own selected tokens (offsets in s_sel)
  uint64_t T = 0;  // partial: the threshold composite
  bool in_lds = false;
  int32_t* row = x.idx + (size_t)x.u * x.ksel;  // the unit's row of idx
  uint32_t* s_sel = x.s_fh;  // (the histogram's room, once the threshold is known)
  __shared__ int s_tok[kFPass];  // a pass's tokens (-1: empty slot)
  __shared__ int s_okl[kFPass];  // its occupied slots

  // ---- the correction's pieces -------------------------------------------------------
  const float sm2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2eF;
  __shared__ float s_qrun[G][kHeadDim / 16];  // sums of 16-channel runs of the query rows
  __shared__ float s_rmh[G];                   // the split's approximate maximum per head
  __shared__ float s_mx[G];
  __shared__ float s_ls[2][G];
  if (tid < G * (kHeadDim / 16)) {
    const int h = tid / (kHeadDim / 16), p = tid % (kHeadDim / 16);
    float r = 0.f;
    for (int c = 0; c < 16; ++c) r += h2f(x.s_q[h][16 * p + c]);
    s_qrun[h][p] = r;
  }
  // key format 2: the query's E2M1 codes as fp16 patterns (value * 2^-14) and
  // 2^(Xq + 28) per 16-channel run; 8 channels per thread, a quad per
  // 32-channel quarter (whole waves)
  constexpr bool kF2 = KF == 2;
  __shared__ uint4 s_q4h[kF2 ? G : 1][kHeadDim / 8];
  __shared__ float s_q4c[kF2 ? G : 1][kHeadDim / 16];
  if constexpr (kF2) {
    if (tid < G * kHeadDim / 8) {
      float xq[8];
      halves8(reinterpret_cast<const uint4*>(&x.s_q[0][0])[tid], xq);
      uint32_t code[8];
      const int X = (int)quantise_lane_e8(xq, code) - 127;
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t c0 = code[2 * j], c1 = code[2 * j + 1];
        pk[j] = ((c0 & 7u) << 9) | ((c0 & 8u) << 12) | ((c1 & 7u) << 25) | ((c1 & 8u) << 28);
      }
      (&s_q4h[0][0])[tid] = (uint4){pk[0], pk[1], pk[2], pk[3]};
      if ((tid & 1) == 0) (&s_q4c[0][0])[tid >> 1] = __builtin_amdgcn_ldexpf(1.0f, X + 28);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int e = tid + NTH * r;
    if ((e & (kHeadDim - 1)) == 0) s_rmh[e / kHeadDim] = rm[r];
  }
  const uint4(*qh)[kHeadDim / 8] = reinterpret_cast<const uint4(*)[kHeadDim / 8]>(&x.s_q[0][0]);
  float(*s_lg)[kFPass][G] = reinterpret_cast<float(*)[kFPass][G]>(x.s_lg);
  float(*s_w)[kFPass][G] = reinterpret_cast<float(*)[kFPass][G]>(x.s_w);
  // the value partial sums of the NW waves: exact in the correction scratch,
  // approximate in the scores' room (both free once the own tokens are known)
  float(*s_pe)[G][kHeadDim] = reinterpret_cast<float(*)[G][kHeadDim]>(x.s_acc);
  float(*s_pa)[G][kHeadDim] = reinterpret_cast<float(*)[G][kHeadDim]>(x.s_split);
  const int tl = tid >> 3, part = tid & 7;  // logits: 8 threads per token
  float ex_m[NR], ex_l[NR], ex_a[NR], ap_l[NR], ap_a[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    ex_m[r] = -INFINITY;
    ex_l[r] = ex_a[r] = ap_l[r] = ap_a[r] = 0.f;
  }
  // One pass over the loads of FPass (tokens toks[j], slot j counted where
  // okv[j] != 0): exact logits and weights (relative to the pass maximum),
  // approximate ones (relative to the split's maximum), the value sums, then
  // the exact state online over the passes and the approximate sums.
  auto pass_run = [&](const FPass<KB, VB, KF>& pd, const int* toks, const int* okv) {
    {
      float ex[G], ap[G];
      run_logits<KB, G, true, true, false, KF>(pd.kr, part, qh, s_qrun, kF2 ? &s_q4h[0] : nullptr, nullptr,
                                               kF2 ? &s_q4c[0] : nullptr, ex, ap);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        ex[h] = sum8(ex[h]);
        ap[h] = sum8(ap[h]);
      }
      if (part == 0) {
        const bool ok = okv[tl] != 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s_lg[0][tl][h] = ok ? ex[h] * sm2 : -INFINITY;
          s_lg[1][tl][h] = ok ? ap[h] * sm2 : -INFINITY;
        }
      }
    }
    __syncthreads();
    // per (exact/approximate, head): lane t of a wave takes slot t -- the
    // weights, their sum and the pass maximum by wave reductions
    for (int cb = wv; cb < 2 * G; cb += NW) {
      const int ty = cb / G, h = cb % G;
      const bool ok = okv[lane] != 0;
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
    {  // lane: channels 2 lane, 2 lane + 1 of the wave's slots 8 wv .. 8 wv + 7
      float pe[G][2], pa[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h) pe[h][0] = pe[h][1] = pa[h][0] = pa[h][1] = 0.f;
      constexpr uint32_t VM = (1u << VB) - 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int slot = 8 * wv + j, t = max(toks[slot], 0);
        int d, bit;
        v_code_pos(VB, t % kTile, 2 * lane, d, bit);
        const half2v_t vh = __builtin_bit_cast(half2v_t, pd.vx[j]);
        const float v0 = (float)vh[0], v1 = (float)vh[1];
        const float sc = h2f((uint16_t)(pd.vm[j] & 0xFFFFu)), zp = h2f((uint16_t)(pd.vm[j] >> 16));
        const float q0 = fmaf(sc, (float)((pd.vd[j][0] >> bit) & VM), zp);
        const float q1 = fmaf(sc, (float)((pd.vd[j][1] >> bit) & VM), zp);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float we = s_w[0][slot][h], wa = s_w[1][slot][h];
          pe[h][0] = fmaf(we, v0, pe[h][0]);
          pe[h][1] = fmaf(we, v1, pe[h][1]);
          pa[h][0] = fmaf(wa, q0, pa[h][0]);
          pa[h][1] = fmaf(wa, q1, pa[h][1]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        *reinterpret_cast<float2*>(&s_pe[wv][h][2 * lane]) = make_float2(pe[h][0], pe[h][1]);
        *reinterpret_cast<float2*>(&s_pa[wv][h][2 * lane]) = make_float2(pa[h][0], pa[h][1]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int e = tid + NTH * r, hh = e / kHeadDim, cc = e & (kHeadDim - 1);
      float pe = 0.f, pa = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        pe += s_pe[w][hh][cc];
        pa += s_pa[w][hh][cc];
      }
      const float mp = s_mx[hh];  // -inf: no counted slot in the pass
      if (mp != -INFINITY) {
        const float mn = fmaxf(ex_m[r], mp);
        const float f0 = __builtin_amdgcn_exp2f(ex_m[r] - mn), f1 = __builtin_amdgcn_exp2f(mp - mn);
        ex_a[r] = fmaf(ex_a[r], f0, pe * f1);
        ex_l[r] = fmaf(ex_l[r], f0, s_ls[0][hh] * f1);
        ex_m[r] = mn;
        ap_a[r] += pa;
        ap_l[r] += s_ls[1][hh];
      }
    }
  };
  auto load_pass = [&](FPass<KB, VB, KF>& pd, const int* toks) {
    pd.load(x.ksh, x.kbase, x.kmeta, x.vsh, x.vbase, x.vmeta, x.cap, x.mshift, toks);
  };

  bool ident = false;  // the selected tokens are the split's offsets 0 .. n_sel - 1
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
    // bin(s) >= Ds  <=>  s >= the least value of bin Ds (the key is monotone
    // in s, -0 and +0 alike): one compare per score instead of its key.
    // Scores are finite or -inf (bin 15); bins 0..14 and above 8176 (+inf)
    // hold only NaN keys, so those Ds take -inf and the least value of 8176.
    constexpr uint32_t kBinNegInf = 15u, kBinPosInf = 8176u;
    const float sth =
        (Ds <= kBinNegInf) ? -INFINITY : key_value(min(Ds, kBinPosInf) << (32 - kFBinBits));
    {
      uint32_t* stage = reinterpret_cast<uint32_t*>(x.s_acc) + wv * kFStage;
      // wave range: a multiple of 256 entries (lane l reads entries 4l..4l+3
      // of each 256 with one 16-byte LDS read; the reads stay inside the
      // kSelStage scores)
      const int R = ((len_s + NW * 256 - 1) / (NW * 256)) * 256;
      const int lo = wv * R, hi = min(len_s, lo + R);
      // (branch-free: the predicates are combined bitwise and a lane with
      // nothing to stage writes its own scratch word -- per-entry branches
      // made this loop several times slower)
      int cnt = 0;
      for (int b0 = lo; b0 < hi; b0 += 512) {
        floatx4 v[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) v[r] = *reinterpret_cast<const floatx4*>(&x.s_split[b0 + 256 * r + 4 * lane]);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int i0 = b0 + 256 * r + 4 * lane;
          int pj[4], c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pj[j] = (int)(i0 + j < hi) & (int)(v[r][j] >= sth);
            c += pj[j];
          }
          const int inc = wave_incl_scan(c);
          int q = cnt + inc - c;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t* dst = (pj[j] & (int)(q < kFStage)) ? &stage[min(q, kFStage - 1)] : &s_junk[lane];
            *dst = (uint32_t)(i0 + j);
            q += pj[j];
          }
          cnt += __builtin_amdgcn_readlane(inc, 63);
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
            len_s, [&](int i) { return x.s_split[i] >= sth; },
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
    // in flight together: the list sizes and bins and the first kBat * 64
    // entries of each wave's first list (whatever its size)
    constexpr int kBat = 8;
    const int q = min(tid, x.nsplit - 1);  // (unconditional loads: a branch around a load waits for it)
    const int lc = (int)ld_dev32(&cnts[q]);
    const uint32_t ld = ld_dev32(&dsv[q]);
    uint64_t lv[kBat];
    {
      const uint64_t* src = lists + (size_t)min(wv, x.nsplit - 1) * x.chunk;
#pragma unroll
      for (int r = 0; r < kBat; ++r) lv[r] = ld_dev64(&src[min(64 * r + lane, x.chunk - 1)]);
    }
    {  // list sizes (prefix sums) and Dmax
      if (tid < x.nsplit) {
        s_dc[tid + 1] = lc;
        atomicMax(&s_dmax, ld);
      }
      __syncthreads();
      if (tid == 0) {
        bool more = x.nsplit > NW;  // entries the first batches do not hold
        s_dc[0] = 0;
        for (int s = 0; s < x.nsplit; ++s) {
          more = more || s_dc[s + 1] > 64 * kBat;
          s_dc[s + 1] += s_dc[s];
        }
        s_n = 0;
        s_more = more ? 1 : 0;
      }
      __syncthreads();
    }
    const uint32_t Dmax = s_dmax;
    const int total = s_dc[x.nsplit];
    in_lds = total <= kFUnion;
    if (in_lds) {
      // the lists to LDS: the first batches from the loads above, the rest
      // (longer lists; splits beyond the first NW) 8 unconditional loads per
      // lane in flight together
      for (int i = tid; i < kFWin; i += NTH) x.s_fh[i] = 0u;
      if (wv < x.nsplit) {
        const int o = s_dc[wv], c = s_dc[wv + 1] - o;
#pragma unroll
        for (int r = 0; r < kBat; ++r) {
          const int p = 64 * r + lane;
          if (p < c) s_union[o + p] = lv[r];
        }
      }
      if (s_more) {
        for (int s = wv; s < x.nsplit; s += NW) {
          const int o = s_dc[s], c = s_dc[s + 1] - o;
          const uint64_t* src = lists + (size_t)s * x.chunk;
          for (int p0 = (s == wv) ? 64 * kBat : 0; p0 < c; p0 += 64 * kBat) {
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
      }
      __syncthreads();
      // every thread keeps its union entries tid + NTH r in registers for
      // the passes below
      constexpr int PU = kFUnion / NTH;
      uint64_t ue[PU];
#pragma unroll
      for (int r = 0; r < PU; ++r) ue[r] = (r < (total + NTH - 1) / NTH) ? s_union[min(tid + NTH * r, total - 1)] : 0ull;
      auto valid = [&](int r) { return tid + NTH * r < total; };
      // their histogram in the bins Dmax .. Dmax + kFWin - 2 (the unit's
      // there; the last counter takes every bin above), then D: thread tid
      // owns counter kFWin - 1 - tid
      const int ru = (total + NTH - 1) / NTH;  // (registers in use: a uniform bound)
#pragma unroll
      for (int r = 0; r < PU; ++r) {
        if (r < ru) {
          const uint32_t b = fbin_c(ue[r]);
          uint32_t* dst = ((int)valid(r) & (int)(b >= Dmax)) ? &x.s_fh[min(b - Dmax, (uint32_t)kFWin - 1)] : &s_junk[lane];
          atomicAdd(dst, 1u);
        }
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
        __syncthreads();
      }
      if (s_res[3]) {  // the kk-th largest lies kFWin - 1 or more bins above Dmax: the full histogram
        for (int i = tid; i < kFBins; i += NTH) x.s_fh[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PU; ++r) {
          const uint32_t b = fbin_c(ue[r]);
          if (valid(r) && b >= Dmax) atomicAdd(&x.s_fh[b], 1u);
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
      } else {
        // a second level inside bin D: the next kFSubBits bits of its
        // entries' composites, histogrammed from the registers; the sub-bin
        // S holding the needD-th largest, then only S's entries are ranked
        constexpr int kSh = 64 - kFBinBits - kFSubBits;
        constexpr int NS = 1 << kFSubBits;
        uint32_t* s_sub = reinterpret_cast<uint32_t*>(x.s_acc);
        for (int i = tid; i < NS; i += NTH) s_sub[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PU; ++r) {
          if (r < ru) {
            uint32_t* dst = ((int)valid(r) & (int)(fbin_c(ue[r]) == D)) ? &s_sub[(uint32_t)(ue[r] >> kSh) & (NS - 1)]
                                                                        : &s_junk[lane];
            atomicAdd(dst, 1u);
          }
        }
        __syncthreads();
        {
          const int mine = (tid < NS) ? (int)s_sub[NS - 1 - tid] : 0;
          int tot;
          const int above = block_excl_scan<NW>(mine, s_wsum, tot);
          if (above < needD && above + mine >= needD) {
            s_res[4] = NS - 1 - tid;
            s_res[5] = above;
            s_res[6] = mine;
          }
          __syncthreads();
        }
        const uint64_t P = ((uint64_t)D << kFSubBits) | (uint64_t)s_res[4];  // the top kFBinBits + kFSubBits bits
        const int needS = needD - s_res[5], inS = s_res[6];
        if (needS == inS) {  // all of sub-bin S
          if (tid == 0) s_T = P << kSh;
        } else if (inS <= NTH) {
          // S's entries to LDS (one atomic per wave and register), then each
          // ranked against all (distinct composites)
          const uint64_t below = (1ull << lane) - 1;
#pragma unroll
          for (int r = 0; r < PU; ++r) {
            const bool p = valid(r) && (ue[r] >> kSh) == P;
            const uint64_t m = __ballot(p);
            if (m) {
              int base = 0;
              if (lane == 0) base = atomicAdd(&s_n, __popcll(m));
              base = __shfl(base, 0);
              if (p) s_dl[base + __popcll(m & below)] = ue[r];
            }
          }
          __syncthreads();
          if (tid < inS) {
            const uint64_t c = s_dl[tid];
            int rk = 0;
            for (int j = 0; j < inS; ++j) rk += (s_dl[j] > c) ? 1 : 0;
            if (rk == needS - 1) s_T = c;
          }
        } else {  // many entries share the top bits (equal scores): radix select among them in LDS
          auto get = [&](int i) -> uint64_t {
            const uint64_t e = s_union[i];
            return (e >> kSh) == P ? e : 0ull;
          };
          const uint64_t t =
              lds_threshold<NTH>(get, total, needS, reinterpret_cast<uint32_t*>(x.s_acc), s_wsum, s_res);
          if (tid == 0) s_T = t;
        }
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
            if (q < kFBins) s_sel[q] = (uint32_t)(t - x.t_begin);
            if (before + q < x.ksel) row[before + q] = t;
          },
          s_wsum);
      if (x.split == 0)
        for (int j = kk + tid; j < x.ksel; j += NTH) row[j] = -1;
    } else {  // (any order; the unit's last workgroup writes idx from the lists)
      if (tid == 0) s_n = 0;
      __syncthreads();
      for (int i = tid; i < len_s; i += NTH)
        if (composite(x.s_split[i], x.t_begin + i) >= T) {
          const int p = atomicAdd(&s_n, 1);
          if (p < kFBins) s_sel[p] = (uint32_t)i;
        }
      __syncthreads();
      n_sel = s_n;
    }
    __syncthreads();
    n_sel = min(min(n_sel, x.ksel), kFBins);  // (<= min(kk, len_s); the clamp only guards the lists)
  } else {
    if (kk > 0) {  // every token is selected
      for (int i = tid; i < len_s; i += NTH) row[x.t_begin + i] = x.t_begin + i;
      n_sel = len_s;
      ident = true;
    }
    if (x.split == 0)
      for (int j = kk + tid; j < x.ksel; j += NTH) row[j] = -1;
    __syncthreads();
  }
  // ---- 3. correction of this split's state ------------------------------------------
  // the selected tokens in passes of kFPass
  for (int p0 = 0; p0 < n_sel; p0 += kFPass) {
    const int np = min(kFPass, n_sel - p0);
    if (tid < kFPass) {
      s_tok[tid] = (tid < np) ? x.t_begin + (ident ? p0 + tid : (int)s_sel[p0 + tid]) : -1;
      s_okl[tid] = (tid < np) ? 1 : 0;
    }
    __syncthreads();
    // (a wave whose 8 slots are all empty loads nothing)
    FPass<KB, VB, KF> pd;
    if (8 * wv < np)
      load_pass(pd, s_tok);
    else
      pd.zero();
    pass_run(pd, s_tok, s_okl);
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
