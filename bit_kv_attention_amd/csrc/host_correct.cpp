// host_correct.cpp -- the exact half of the correction on the host's cores,
// from a host-resident fp16 copy of the cache (JetFire README, introduction:
// "Approximate-then-Correct Attention on Hybrid Memory" -- the low-bit cache
// is attended on the GPU and the top-k tokens are corrected from the
// high-precision copy kept in host memory).
//
// For every (b, query head h) and the selected set S of its KV head:
//   lambda_t = log2(e) / sqrt(D) * q_h . K_t            (log2 units, t in S)
//   m = max_S lambda_t,  l = sum_S 2^(lambda_t - m),  a = sum_S 2^(lambda_t - m) V_t
// stored as {m, l, a[0..D)}: the exact record qattn_correct_hybrid merges with
// the GPU's approximate state.  Products and sums in fp32 (the GPU's exact
// path uses the same precision).
//
// Units (b, kvh) are spread over OpenMP threads.  Tokens go in runs of 64:
// the run's logits, its maximum, a rescale of the running sums, then the
// run's values, so nothing is allocated whatever k is; a run's scattered rows
// are prefetched together before they are used.  The x86 path uses
// AVX2/FMA/F16C (16-byte half loads converted in registers); machines without
// them take the plain loop.
#include <immintrin.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include "bitkv.h"

namespace {

constexpr int kD = 128;
constexpr int kGroupSize = 32;
constexpr int kState = 2 + kD;
constexpr int kRun = 64;
constexpr int kMaxG = 8;

float half_bits_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu, bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal: m * 2^-24, normalised
      int sh = 0;
      while (!(m & 0x400u)) {
        m <<= 1;
        ++sh;
      }
      bits = sign | ((uint32_t)(113 - sh) << 23) | ((m & 0x3FFu) << 13);
    }
  } else if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

struct UnitArgs {
  const uint16_t* ksh;  // the unit's shadow rows [cap][D]
  const uint16_t* vsh;
  const uint16_t* q;    // the G query rows [G][D]
  const int32_t* sel;   // k row entries
  int k, n, G;
  float* out;           // [G][kState]
};

// Rows as floats: the portable path converts one value at a time.
struct PlainRows {
  static void row(const uint16_t* h, float* f) {
    for (int c = 0; c < kD; ++c) f[c] = half_bits_to_float(h[c]);
  }
  static float dot(const float* a, const float* b) {
    float s = 0.f;
    for (int c = 0; c < kD; ++c) s += a[c] * b[c];
    return s;
  }
  static void axpy(float w, const float* x, float* y) {
    for (int c = 0; c < kD; ++c) y[c] += w * x[c];
  }
};

struct Avx2Rows {
  __attribute__((target("avx2,fma,f16c"))) static void row(const uint16_t* h, float* f) {
    for (int c = 0; c < kD; c += 8)
      _mm256_storeu_ps(f + c, _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(h + c))));
  }
  __attribute__((target("avx2,fma,f16c"))) static float dot(const float* a, const float* b) {
    __m256 s0 = _mm256_setzero_ps(), s1 = _mm256_setzero_ps();
    for (int c = 0; c < kD; c += 16) {
      s0 = _mm256_fmadd_ps(_mm256_loadu_ps(a + c), _mm256_loadu_ps(b + c), s0);
      s1 = _mm256_fmadd_ps(_mm256_loadu_ps(a + c + 8), _mm256_loadu_ps(b + c + 8), s1);
    }
    const __m256 s = _mm256_add_ps(s0, s1);
    __m128 x = _mm_add_ps(_mm256_castps256_ps128(s), _mm256_extractf128_ps(s, 1));
    x = _mm_add_ps(x, _mm_movehl_ps(x, x));
    x = _mm_add_ss(x, _mm_shuffle_ps(x, x, 1));
    return _mm_cvtss_f32(x);
  }
  __attribute__((target("avx2,fma,f16c"))) static void axpy(float w, const float* x, float* y) {
    const __m256 wv = _mm256_set1_ps(w);
    for (int c = 0; c < kD; c += 8)
      _mm256_storeu_ps(y + c, _mm256_fmadd_ps(wv, _mm256_loadu_ps(x + c), _mm256_loadu_ps(y + c)));
  }
};

template <class R>
inline __attribute__((always_inline)) void unit_state(const UnitArgs& a) {
  const float sm2 = 1.4426950408889634f / sqrtf((float)kD);
  float q[kMaxG][kD], acc[kMaxG][kD], m[kMaxG], l[kMaxG];
  float lam[kMaxG][kRun], f[kD];
  int ts[kRun];
  for (int h = 0; h < a.G; ++h) {
    R::row(a.q + (size_t)h * kD, q[h]);
    for (int c = 0; c < kD; ++c) acc[h][c] = 0.f;
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  const int kk = a.k < a.n ? a.k : a.n;  // entries past min(k, len) are not read
  int i = 0;
  while (i < kk) {
    int cnt = 0;  // the next run of valid entries
    for (; i < kk && cnt < kRun; ++i) {
      const int t = a.sel[i];
      if (t >= 0 && t < a.n) ts[cnt++] = t;
    }
    if (cnt == 0) break;
    // the run's rows are scattered 256-byte records: request them all before
    // the first is used, so the memory system works on them together
    for (int j = 0; j < cnt; ++j)
      for (int x = 0; x < kD * 2; x += 64) {
        __builtin_prefetch(reinterpret_cast<const char*>(a.ksh + (size_t)ts[j] * kD) + x, 0, 3);
        __builtin_prefetch(reinterpret_cast<const char*>(a.vsh + (size_t)ts[j] * kD) + x, 0, 3);
      }
    for (int j = 0; j < cnt; ++j) {
      R::row(a.ksh + (size_t)ts[j] * kD, f);
      for (int h = 0; h < a.G; ++h) lam[h][j] = sm2 * R::dot(q[h], f);
    }
    float sc[kMaxG];
    for (int h = 0; h < a.G; ++h) {
      float mx = m[h];
      for (int j = 0; j < cnt; ++j) mx = lam[h][j] > mx ? lam[h][j] : mx;
      sc[h] = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - mx);
      m[h] = mx;
      l[h] *= sc[h];
      for (int c = 0; c < kD; ++c) acc[h][c] *= sc[h];
    }
    for (int j = 0; j < cnt; ++j) {
      R::row(a.vsh + (size_t)ts[j] * kD, f);
      for (int h = 0; h < a.G; ++h) {
        const float w = exp2f(lam[h][j] - m[h]);
        l[h] += w;
        R::axpy(w, f, acc[h]);
      }
    }
  }
  for (int h = 0; h < a.G; ++h) {
    float* o = a.out + (size_t)h * kState;
    o[0] = m[h];
    o[1] = l[h];
    for (int c = 0; c < kD; ++c) o[2 + c] = acc[h][c];
  }
}

__attribute__((target("avx2,fma,f16c"))) void unit_state_avx2(const UnitArgs& a) { unit_state<Avx2Rows>(a); }

bkv_status check(const bkv_layout* L) {
  if (!L) return BKV_E_NULL;
  if (L->batch <= 0 || L->n_q_heads <= 0 || L->n_kv_heads <= 0 || L->head_dim <= 0 || L->group <= 0 ||
      L->capacity <= 0 || L->n_q_heads % L->n_kv_heads != 0 || L->head_dim % L->group != 0 || L->capacity % 32 != 0)
    return BKV_E_SHAPE;
  const int G = L->n_q_heads / L->n_kv_heads;
  if (L->head_dim != kD || (L->group != kGroupSize && L->group != 2 * kGroupSize) || L->k_bits < 1 || L->k_bits > 4 ||
      (L->v_bits != 2 && L->v_bits != 4) || (G != 4 && G != 8) || L->batch > 256)
    return BKV_E_UNSUPPORTED;
  return BKV_OK;
}

}  // namespace

extern "C" bkv_status qattn_exact_host(const bkv_layout* L, const uint16_t* k_shadow, const uint16_t* v_shadow,
                                       const uint16_t* q, const int32_t* len_host, const int32_t* idx, int32_t k,
                                       float* state, int32_t n_threads) {  // (host pointers throughout)
  bkv_status st = check(L);
  if (st != BKV_OK) return st;
  if (k < 0 || n_threads < 0) return BKV_E_ARG;
  if (!k_shadow || !v_shadow || !q || !len_host || !state || (!idx && k > 0)) return BKV_E_NULL;
  for (int b = 0; b < L->batch; ++b)
    if (len_host[b] < 0 || len_host[b] > L->capacity) return BKV_E_CAPACITY;
  const int G = L->n_q_heads / L->n_kv_heads;
  const int units = L->batch * L->n_kv_heads;
  const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c");
  const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int b = u / L->n_kv_heads;
    UnitArgs a;
    a.ksh = k_shadow + (size_t)u * L->capacity * kD;
    a.vsh = v_shadow + (size_t)u * L->capacity * kD;
    a.q = q + (size_t)u * G * kD;  // query heads u*G .. u*G + G - 1 of [B][Hq]
    a.sel = k > 0 ? idx + (size_t)u * k : nullptr;
    a.k = k;
    a.n = len_host[b];
    a.G = G;
    a.out = state + (size_t)u * G * kState;
    if (avx2)
      unit_state_avx2(a);
    else
      unit_state<PlainRows>(a);
  }
  return BKV_OK;
}
