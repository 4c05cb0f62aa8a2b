// hybrid_layers.hip -- the hybrid step over several layers, scheduled on the
// host (JetFire README, introduction: a low-bit cache on the GPU and the
// high-precision correction of the top-k tokens on the host, "on hybrid
// memory").  Host code only: it calls the library's own entry points.
//
// A layer's query depends on the previous layer's output, so the host pass
// of one layer cannot overlap the next layer's scan of the same sequences.
// The batch is split into `micro` micro-batches of consecutive batch rows;
// while the host computes micro-batch m's exact states of layer i, the GPU
// runs what is queued for the others.  Per micro-batch and layer, on the
// caller's stream: qattn_decode_step (append, scan, top-k), the copies of
// the rows and of the query to the slot's pinned host buffers, an event.
// The host waits for that event only, runs qattn_exact_host, then enqueues
// the copy of the states to the device, qattn_correct_hybrid into the
// layer's output and the micro-batch's next layer.  A micro-batch's slot is
// reused only after its previous merge is queued, and everything of one
// micro-batch is on the one stream, so the GPU keeps their order.
#include <string.h>

#include "bkv_internal.h"

using namespace bkv;

extern "C" {

bkv_status qattn_hybrid_layers(const bkv_layout* L, int32_t n_layers, const bkv_cache* caches,
                               const uint16_t* const* q, const uint16_t* const* k_new,
                               const uint16_t* const* v_new, const int32_t* pos_host, int32_t k, int32_t micro,
                               const bkv_hybrid_slot* slots, float* const* out, int32_t n_threads, void* stream) {
  if (!L || !caches || !q || !k_new || !v_new || !pos_host || !slots || !out) return BKV_E_NULL;
  if (n_layers < 0 || k < 0 || n_threads < 0 || micro < 1 || L->batch % micro != 0) return BKV_E_ARG;
  if (n_layers == 0) return BKV_OK;
  const int nb = L->batch / micro;
  bkv_layout lm = *L;
  lm.batch = nb;
  // the whole call is validated before anything is enqueued: the positions,
  // every slot's workspace (for the call's longest length) and every layer's
  // pointers
  int max_len = 0;
  for (int b = 0; b < L->batch; ++b) {
    if (pos_host[b] < 0 || pos_host[b] >= L->capacity) return BKV_E_CAPACITY;
    max_len = pos_host[b] + 1 > max_len ? pos_host[b] + 1 : max_len;
  }
  size_t ws_need = 0;
  bkv_status st = bkv_workspace_bytes(&lm, max_len, k, &ws_need);
  if (st != BKV_OK) return st;
  for (int m = 0; m < micro; ++m) {
    const bkv_hybrid_slot& s = slots[m];
    if (!s.sigma || !s.ws || !s.state_dev || !s.q_host || !s.state_host || (k > 0 && (!s.idx || !s.idx_host)))
      return BKV_E_NULL;
    if (s.ws_bytes < ws_need) return BKV_E_WORKSPACE;
  }
  for (int i = 0; i < n_layers; ++i) {
    const bkv_cache& c = caches[i];
    if (!c.k_codes || !c.v_codes || !c.k_meta || !c.v_meta || !c.k_shadow || !c.v_shadow || !q[i] || !k_new[i] ||
        !v_new[i] || !out[i])
      return BKV_E_NULL;
  }
  int32_t lens[kMaxBatch];
  for (int b = 0; b < L->batch; ++b) lens[b] = pos_host[b] + 1;

  const size_t units_m = (size_t)nb * L->n_kv_heads;
  size_t kcb = 0, vcb = 0, mb = 0, sb = 0, kmb = 0;
  if ((st = bkv_cache_bytes(L, &kcb, &vcb, &mb, &sb)) != BKV_OK) return st;
  if ((st = bkv_k_meta_bytes(L, &kmb)) != BKV_OK) return st;
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  // bytes per unit of each buffer: micro-batch m's views start at unit m * units_m
  const size_t pu_kc = kcb / units, pu_vc = vcb / units, pu_km = kmb / units, pu_vm = mb / units, pu_sh = sb / units;
  const size_t per_q = (size_t)nb * L->n_q_heads * L->head_dim;
  const size_t per_kv = (size_t)nb * L->n_kv_heads * L->head_dim;
  const hipStream_t s = (hipStream_t)stream;

  auto view = [&](int i, int m) {
    const bkv_cache& c = caches[i];
    const size_t u0 = (size_t)m * units_m;
    bkv_cache v;
    v.k_codes = static_cast<char*>(c.k_codes) + u0 * pu_kc;
    v.v_codes = static_cast<char*>(c.v_codes) + u0 * pu_vc;
    v.k_meta = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(c.k_meta) + u0 * pu_km);
    v.v_meta = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(c.v_meta) + u0 * pu_vm);
    v.k_shadow = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(c.k_shadow) + u0 * pu_sh);
    v.v_shadow = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(c.v_shadow) + u0 * pu_sh);
    return v;
  };

  hipEvent_t ev[kMaxBatch];
  int made = 0;
  bkv_status res = BKV_OK;
  for (; made < micro; ++made)
    if (hipEventCreateWithFlags(&ev[made], hipEventDisableTiming) != hipSuccess) {
      res = BKV_E_HIP;
      break;
    }
  // micro-batch m, layer i: append, scan, top-k, rows and query to the host
  auto select = [&](int i, int m) -> bkv_status {
    const bkv_hybrid_slot& sl = slots[m];
    const bkv_cache v = view(i, m);
    bkv_status r = qattn_decode_step(&lm, &v, k_new[i] + m * per_kv, v_new[i] + m * per_kv, q[i] + m * per_q,
                                     lens + m * nb, k, sl.sigma, sl.idx, sl.ws, sl.ws_bytes, 0, stream);
    if (r != BKV_OK) return r;
    if (k > 0 && hipMemcpyAsync(sl.idx_host, sl.idx, units_m * k * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
                     hipSuccess)
      return BKV_E_HIP;
    if (hipMemcpyAsync(sl.q_host, q[i] + m * per_q, per_q * sizeof(uint16_t), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
      return BKV_E_HIP;
    return hipEventRecord(ev[m], s) == hipSuccess ? BKV_OK : BKV_E_HIP;
  };
  for (int m = 0; res == BKV_OK && m < micro; ++m) res = select(0, m);
  const size_t state_bytes = (size_t)nb * L->n_q_heads * (L->head_dim + 2) * sizeof(float);
  for (int i = 0; res == BKV_OK && i < n_layers; ++i) {
    for (int m = 0; res == BKV_OK && m < micro; ++m) {
      const bkv_hybrid_slot& sl = slots[m];
      const bkv_cache v = view(i, m);
      if (hipEventSynchronize(ev[m]) != hipSuccess) {  // this micro-batch's rows, query and new token
        res = BKV_E_HIP;
        break;
      }
      res = qattn_exact_host(&lm, v.k_shadow, v.v_shadow, sl.q_host, lens + m * nb, sl.idx_host, k, sl.state_host,
                             n_threads);
      if (res != BKV_OK) break;
      if (hipMemcpyAsync(sl.state_dev, sl.state_host, state_bytes, hipMemcpyHostToDevice, s) != hipSuccess) {
        res = BKV_E_HIP;
        break;
      }
      res = qattn_correct_hybrid(&lm, &v, q[i] + m * per_q, lens + m * nb, k > 0 ? sl.idx : nullptr, k,
                                 sl.state_dev, sl.ws, sl.ws_bytes, out[i] + m * per_q, stream);
      if (res == BKV_OK && i + 1 < n_layers) res = select(i + 1, m);
    }
  }
  for (int m = 0; m < made; ++m) (void)hipEventDestroy(ev[m]);
  return res;
}

}  // extern "C"
