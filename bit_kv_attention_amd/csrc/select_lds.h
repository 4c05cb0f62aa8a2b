// select_lds.h -- workgroup-wide selection of the need-th largest composite
// (score, index) key, and the merge of per-slice candidates, shared by the
// top-k kernels and the scan's in-launch selection.
//
// A token's composite key is (order-preserving bits of its score) << 32 | ~t:
// larger means a larger score, or an equal score and a lower index, and no
// two tokens share one.  hist_select (below) finds the need-th largest T with
// one histogram of score values and an exact ranking of the threshold bin.
// lds_threshold is the general radix select it falls back on: most
// significant digit first (widths 12, 10, 10 over the score bits, 11, 11, 10
// over the index bits), a pass histograms the next digit of the entries under
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

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within
// each row of 16 lanes, then lane 15 of rows 0 and 2 is added into rows 1 and
// 3 and lane 31 into rows 2 and 3 (row broadcasts).  Lanes without a source
// add 0.
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Minimum / maximum over the 64 lanes of a wave, in every lane: DPP within a
// row, then the gfx950 row swaps (each returns own and partner value).
template <bool MAX>
__device__ inline float wave_minmax(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));   // quad [1,0,3,2]
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));   // quad [2,3,0,1]
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true)));  // row_ror:4
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true)));  // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Exclusive prefix sum over a workgroup of NW waves (wave scan, then the wave
// totals through LDS); `total` gets the sum of all.
template <int NW>
__device__ inline int block_excl_scan(int v, int* s_wsum, int& total) {
  const int lane = (int)__builtin_amdgcn_workitem_id_x() & 63, wv = (int)__builtin_amdgcn_workitem_id_x() >> 6;
  const int x = wave_incl_scan(v);
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
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
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

namespace bkv {

// Value of a float_key (-0 comes back as +0).
__device__ inline float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

constexpr int kHistBins = 4096;

// The need-th largest of the composites spread over the workgroup, with few
// barriers.  Each thread holds PER entries in c[] (0 = empty slot; which
// entries, does not matter here).  One histogram of the score values over
// kHistBins equal bins between the smallest and largest score -- the bin is
// monotone in the score, so every entry of a higher bin beats every entry of
// a lower one; one scan finds the bin D holding the need-th largest, and the
// entries of bin D are ranked exactly: by one wave when at most 64 (the
// usual case: the bins are narrow), else by the radix select restricted to
// bin D, for which fill() first puts every entry i of [0, count) where get(i)
// reads it.  s_hist: kHistBins words; s_mm: 2*NT/64 floats; s_small: 65
// words; s_res: 4 ints.
template <int NT, int PER, typename Get, typename Fill>
__device__ inline uint64_t hist_select(const uint64_t (&c)[PER], int count, int need, Get get, Fill fill,
                                       uint32_t* s_hist, int* s_wsum, int* s_res, float* s_mm, uint64_t* s_small) {
  constexpr int NW = NT / 64;
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const float x = key_value((uint32_t)(c[j] >> 32));
    lo = c[j] ? fminf(lo, x) : lo;
    hi = c[j] ? fmaxf(hi, x) : hi;
  }
  lo = wave_minmax<false>(lo);
  hi = wave_minmax<true>(hi);
  for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
  if (lane == 0) {
    s_mm[wv] = lo;
    s_mm[NW + wv] = hi;
  }
  if (tid == 0) s_res[2] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = fminf(lo, s_mm[w]);
    hi = fmaxf(hi, s_mm[NW + w]);
  }
  // bin(x) = clamp(floor((x - lo) * scale)): monotone in x (each step is);
  // an empty or infinite range puts everything in one bin (fmaxf drops NaN)
  const float scale = (float)kHistBins / (hi - lo);
  auto bin = [&](uint64_t cc) {
    const float f = (key_value((uint32_t)(cc >> 32)) - lo) * scale;
    return (int)fminf(fmaxf(f, 0.0f), (float)(kHistBins - 1));
  };
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (c[j]) atomicAdd(&s_hist[bin(c[j])], 1u);
  __syncthreads();
  // the bin D with  sum_{x > D} hist[x] < need <= sum_{x >= D} hist[x]
  constexpr int per = kHistBins / NT;
  const int top = kHistBins - 1 - tid * per;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) mine += (int)s_hist[top - i];
  int total;
  int above = block_excl_scan<NW>(mine, s_wsum, total);
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
  const int need2 = need - s_res[1];
  const int mD = (int)s_hist[D];
  if (mD > 64) {  // many entries share bin D: radix select among them
    fill();
    __syncthreads();  // s_hist is reused; the entries are in place
    auto getD = [&](int i) {
      const uint64_t cc = get(i);
      return (cc && bin(cc) == D) ? cc : 0ull;
    };
    return lds_threshold<NT>(getD, count, need2, s_hist, s_wsum, s_res);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (c[j] && bin(c[j]) == D) s_small[atomicAdd(&s_res[2], 1)] = c[j];
  __syncthreads();
  if (wv == 0) {  // rank the (distinct) entries of bin D
    const uint64_t x = lane < mD ? s_small[lane] : 0ull;
    int rank = 0;
    for (int i = 0; i < mD; ++i) rank += s_small[i] > x ? 1 : 0;
    if (lane < mD && rank == need2 - 1) s_small[64] = x;
  }
  __syncthreads();
  return s_small[64];
}

// Entries [kk, stride) of a unit's row: the nw window tokens n, n+1, ...,
// then -1.  All NT threads of the workgroup.
template <int NT>
__device__ inline void write_tail(int32_t* __restrict__ out, int kk, int n, int nw, int stride) {
  for (int i = (int)__builtin_amdgcn_workitem_id_x(); i < stride - kk; i += NT) out[kk + i] = (i < nw) ? n + i : -1;
}

// Data crosses workgroups of one launch only through agent-scope atomic
// stores, loads and read-modify-writes.  gfx950 performs those at the
// device's coherence point: they do not stay in (or read from) an XCD's own
// L2, which the other XCDs do not see.  A workgroup hands data over by
// waiting in every wave until its own atomic stores are performed
// (s_waitcnt vmcnt(0)), then -- after a barrier -- incrementing a counter;
// a receiver issues its atomic loads only after it has read the count.  No
// cache-wide release or acquire is needed for data that never sits in a
// non-coherent cache, and none is taken: on this device an agent-scope
// release fence writes back the XCD's whole L2 and an acquire fence
// invalidates it, which measured several microseconds per arrival.
__device__ inline void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t ld_dev32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_devf(float* p, float v) { st_dev32(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
__device__ inline float ld_devf(const float* p) { return __uint_as_float(ld_dev32(reinterpret_cast<const uint32_t*>(p))); }

// Every wave waits until its memory operations are performed, then the
// workgroup meets at a barrier (the builtin wait is a scheduling barrier for
// the compiler too).
__device__ inline void wg_drain() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Arrival of a workgroup at a counter shared by the n workgroups of a unit;
// true (in every thread) in the workgroup that brings it to n.  What the
// workgroups stored with st_dev* before arriving, the last one reads with
// ld_dev* after.
__device__ inline bool arrive_is_last(uint32_t* ctr, uint32_t n, int* s_flag) {
  wg_drain();
  if (__builtin_amdgcn_workitem_id_x() == 0)
    *s_flag = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  __syncthreads();
  return *s_flag != 0;
}

// A barrier across the n workgroups of a unit within one launch (they are
// all resident: the launcher checks that the grid fits the device at once).
// After arriving, one thread polls the counter until it reads n.  The poll
// is bounded (kSpinMax polls of about 64 clocks each plus the load, on the
// order of a second): past it the flag word gets bit 0 and the workgroup goes
// on, so a launch always ends.  The counter is left at n; the unit's last
// workgroup of the launch resets it.
constexpr int kSpinMax = 1 << 20;
__device__ inline void unit_barrier(uint32_t* ctr, uint32_t n, uint32_t* flag) {
  wg_drain();
  if (__builtin_amdgcn_workitem_id_x() == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0;; ++it) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) break;
      if (it == kSpinMax) {
        __hip_atomic_fetch_or(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Output positions of the selected entries held as entry j*NW*64 + 64w + lane
// (wave w): their rank in that order among the selected ones.  Per (j, w) the
// count comes from a ballot, one block scan over the PER*NW counts places
// them.  s_tmp: PER*NW ints.
template <int PER, int NW>
__device__ inline void ordered_positions(const bool (&sel)[PER], int (&at)[PER], int* s_wsum, int* s_tmp,
                                         int* total_out = nullptr) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63, wv = tid >> 6;
  const uint64_t below = (1ull << lane) - 1;
  uint64_t mask[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    mask[j] = __ballot(sel[j]);
    if (lane == 0) s_tmp[j * NW + wv] = __popcll(mask[j]);
  }
  __syncthreads();
  const int cnt = (tid < PER * NW) ? s_tmp[tid] : 0;
  int total;
  const int before = block_excl_scan<NW>(cnt, s_wsum, total);  // (its barriers order the reads above)
  if (total_out) *total_out = total;
  if (tid < PER * NW) s_tmp[tid] = before;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) at[j] = s_tmp[j * NW + wv] + __popcll(mask[j] & below);
}

// The merge of one unit's candidate slots: slice s of S tokens left its
// top-min(k, slice length) composites in index order at ucand[s*k ..], 0 in
// its unused slots.  The kk = min(k, n)-th largest slot is found and the slots
// >= it are written in slot order, which is ascending token order, to the
// unit's row of k + W entries, then the window and -1 (write_tail).  All NT
// threads.  AGENT: the slots were written by other workgroups of this launch.
// At most MAXSLOTS slots.  n: tokens selected from (the window's nw follow).
template <int NT, bool AGENT, int MAXSLOTS>
__device__ __attribute__((always_inline)) inline void merge_unit(const uint64_t* __restrict__ ucand, int32_t* __restrict__ idx, int u, int n, int nw,
                           int k, int W, int S, uint64_t* s_c, uint32_t* s_hist, int* s_wsum, int* s_res, float* s_mm,
                           uint64_t* s_small) {
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int kk = min(k, n);
  int32_t* __restrict__ out = idx + (size_t)u * (k + W);
  write_tail<NT>(out, kk, n, nw, k + W);
  if (kk == n || kk == 0) {  // every token (or none) is selected
    for (int i = tid; i < kk; i += NT) out[i] = i;
  } else {
    const int ns = (n + S - 1) / S;  // slices holding tokens
    const int slots = ns * k;
    // thread tid holds slots j*NT + tid (coalesced loads)
    constexpr int kPer = MAXSLOTS / NT;
    uint64_t v[kPer];  // 0: empty
    bool ok[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {  // clamped, unconditional loads first (unused slots hold 0)
      const int p = j * NT + tid;
      const uint64_t* src = &ucand[min(p, slots - 1)];
      v[j] = AGENT ? ld_dev64(src) : *src;
      ok[j] = p < slots;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = ok[j] ? v[j] : 0;
    auto get = [&](int i) { return s_c[i]; };
    auto fill = [&]() {
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (j * NT + tid < slots) s_c[j * NT + tid] = v[j];
    };
    const uint64_t T = hist_select<NT>(v, slots, kk, get, fill, s_hist, s_wsum, s_res, s_mm, s_small);
    // the slots >= T in slot order (ascending token order): slot j*NT +
    // 64w + lane is (j, w, lane) in that order
    bool sel[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) sel[j] = v[j] && v[j] >= T;
    int at[kPer];
    ordered_positions<kPer, NT / 64>(sel, at, s_wsum, reinterpret_cast<int*>(s_hist));
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (sel[j]) out[at[j]] = (int32_t)~(uint32_t)(v[j] & 0xFFFFFFFFu);
  }
}

}  // namespace bkv
