"""One decode step = the four C-ABI calls on one stream, with the buffers they
need allocated once (torch device memory).  Marshalling only."""
from __future__ import annotations

from . import binding as bk


class DecodeStep:
    """Buffers for steps of one layer shape: sigma, workspace, idx, out.
    window > 0 also corrects the newest `window` tokens of every sequence
    (topk_select_window); the rows of idx then hold k + window entries.
    block > 0 selects k whole blocks of `block` tokens instead
    (topk_select_blocks); the rows then hold k * block entries.  Plain top-k
    runs as qattn_decode_select with select_mode (automatic: the selection in
    the scan's launch where that is faster) unless fused is False, which makes
    the two calls qattn_decode_approx and topk_select.  one_launch runs the
    plain top-k step as qattn_decode_fused: scan, selection and correction in
    one launch (falling back to the separate launches for a call the library
    cannot run that way)."""

    def __init__(self, layout: bk.Layout, k: int, max_len: int, device="cuda", window: int = 0, block: int = 0,
                 fused: bool = True, select_mode: int = bk.SELECT_AUTO, exclude: bool | None = None,
                 one_launch: bool | None = None):
        import torch
        self.fused = bool(fused)
        # exclude: a second approximate pass over the unselected tokens, merged
        # with the selected tokens' exact terms instead of subtracting their
        # approximate ones (default for 1- and 2-bit keys, whose approximate
        # logits can overshoot by far more than fp32 subtraction survives)
        self.exclude = (layout.k_bits <= 2) if exclude is None else bool(exclude)
        self.select_mode = int(select_mode)
        self.layout = layout
        self.k = int(k)
        self.window = int(window)
        self.block = int(block)
        if self.block and self.window:
            raise ValueError("a recent window and block selection do not combine")
        self.row = self.k * self.block if self.block else self.k + self.window
        L = layout
        self.sigma = torch.empty(L.batch * L.n_kv_heads * L.capacity, dtype=torch.float32, device=device)
        ws_bytes = bk.bkv_workspace_bytes(L, max_len, self.row)
        # zero-filled once: the calls keep their arrival counters in it at zero
        self.ws = torch.zeros(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device=device)
        self.idx = torch.empty(L.batch * L.n_kv_heads * max(self.row, 1), dtype=torch.int32, device=device)
        self.out = torch.empty(L.batch * L.n_q_heads * L.head_dim, dtype=torch.float32, device=device)
        plain = self.fused and not self.exclude and self.block == 0 and self.window == 0
        if one_launch is None:  # (opt-in while the separate launches are faster)
            one_launch = False
        elif one_launch and not plain:
            raise ValueError("one_launch runs the plain top-k step only")
        self.one_launch = bool(one_launch)
        self.ran_fused = False  # whether the last call ran as one launch

    def attend(self, cache: bk.Cache, q, lens, stream=None):
        """Approximate pass, top-k, exact correction over the first lens[b] tokens."""
        if self.exclude:
            return self._attend_exclude(cache, q, lens, stream)
        if self.one_launch and self._fused(cache, None, None, q, lens, stream):
            return self.out
        if self.fused and self.block == 0 and self.window == 0:
            bk.qattn_decode_select(self.layout, cache, q, lens, self.k, self.sigma, self.idx, self.ws, stream,
                                   self.select_mode)
            bk.qattn_correct(self.layout, cache, q, lens, self.idx if self.k > 0 else None, self.k, self.ws,
                             self.out, stream)
            return self.out
        bk.qattn_decode_approx(self.layout, cache, q, lens, self.sigma, self.ws, stream)
        if self.block > 0:
            if self.k > 0:
                bk.topk_select_blocks(self.layout, self.sigma, lens, self.k, self.block, self.idx, self.ws, stream)
            bk.qattn_correct_blocks(self.layout, cache, q, lens, self.idx if self.k > 0 else None, self.k, self.block,
                                    self.ws, self.out, stream)
            return self.out
        elif self.window > 0:
            bk.topk_select_window(self.layout, self.sigma, lens, self.k, self.window, self.idx, self.ws, stream)
        elif self.k > 0:
            bk.topk_select(self.layout, self.sigma, lens, self.k, self.idx, self.ws, stream)
        bk.qattn_correct(self.layout, cache, q, lens, self.idx if self.row > 0 else None, self.row, self.ws,
                         self.out, stream)
        return self.out

    def _fused(self, cache, k_new, v_new, q, lens, stream) -> bool:
        """qattn_decode_fused; False (nothing enqueued) when the library cannot
        run this call in one launch (e.g. the device cannot hold its grid)."""
        self.ran_fused = False
        try:
            bk.qattn_decode_fused(self.layout, cache, k_new, v_new, q, lens, self.k, self.sigma,
                                  self.idx if self.k > 0 else None, self.out, self.ws, stream)
        except bk.BitKVError as e:
            if e.status != 3:  # BKV_E_UNSUPPORTED
                raise
            return False
        self.ran_fused = True
        return True

    def _attend_exclude(self, cache: bk.Cache, q, lens, stream=None):
        if self.block > 0:
            bk.qattn_decode_approx(self.layout, cache, q, lens, self.sigma, self.ws, stream)
            if self.k > 0:
                bk.topk_select_blocks(self.layout, self.sigma, lens, self.k, self.block, self.idx, self.ws, stream)
        elif self.window > 0:
            bk.qattn_decode_approx(self.layout, cache, q, lens, self.sigma, self.ws, stream)
            bk.topk_select_window(self.layout, self.sigma, lens, self.k, self.window, self.idx, self.ws, stream)
        else:  # scores and rows only: the state comes from the second pass
            bk.qattn_score_select(self.layout, cache, q, lens, self.k, self.sigma, self.idx, self.ws, stream,
                                  self.select_mode)
        idx = self.idx if self.row > 0 else None
        bk.qattn_decode_unselected(self.layout, cache, q, lens, idx, self.row, self.ws, stream)
        bk.qattn_correct_unselected(self.layout, cache, q, lens, idx, self.row, self.ws, self.out, stream)
        return self.out

    def attend_hybrid(self, cache: bk.Cache, q, lens, n_threads: int = 0, select: bool = True):
        """The same step with the exact half of the correction on the host
        (qattn_exact_host over the cache's pinned host shadow), merged on the
        GPU by qattn_correct_hybrid.  Synchronises the current stream once, to
        hand the selected rows to the host."""
        import torch
        if cache.k_shadow.is_cuda:
            raise ValueError("attend_hybrid needs a cache with its shadow in host memory")
        if self.exclude:
            raise ValueError("attend_hybrid subtracts the selected tokens' approximate terms, which 1- and 2-bit "
                             "keys do not survive in fp32: use attend()")
        if not hasattr(self, "_h_idx"):
            L = self.layout
            self._h_idx = torch.empty(self.idx.numel(), dtype=torch.int32, pin_memory=True)
            self._h_q = torch.empty(L.batch * L.n_q_heads * L.head_dim, dtype=torch.float16, pin_memory=True)
            self._h_state = torch.empty(L.batch * L.n_q_heads * (L.head_dim + 2), dtype=torch.float32,
                                        pin_memory=True)
            self._d_state = torch.empty_like(self._h_state, device=self.out.device)
        if select:  # else the caller has run qattn_decode_select for this step
            bk.qattn_decode_select(self.layout, cache, q, lens, self.k, self.sigma, self.idx, self.ws,
                                   mode=self.select_mode)
        self._h_idx.copy_(self.idx, non_blocking=True)
        self._h_q.copy_(q.reshape(-1), non_blocking=True)
        torch.cuda.current_stream().synchronize()
        bk.qattn_exact_host(self.layout, cache.k_shadow, cache.v_shadow, self._h_q, lens, self._h_idx, self.k,
                            self._h_state, n_threads)
        self._d_state.copy_(self._h_state, non_blocking=True)
        bk.qattn_correct_hybrid(self.layout, cache, q, lens, self.idx if self.k > 0 else None, self.k,
                                self._d_state, self.ws, self.out)
        return self.out

    def step(self, cache: bk.Cache, q, k_new, v_new, pos, stream=None):
        """Append one token per sequence at pos[b], then attend over pos[b] + 1
        tokens.  The plain top-k step appends inside the scan's launch
        (qattn_decode_step)."""
        lens = [int(p) + 1 for p in pos]
        if self.one_launch and self._fused(cache, k_new, v_new, q, lens, stream):
            return self.out
        if self.fused and not self.exclude and self.block == 0 and self.window == 0 and min(lens) >= 1:
            bk.qattn_decode_step(self.layout, cache, k_new, v_new, q, lens, self.k, self.sigma, self.idx, self.ws,
                                 stream, self.select_mode)
            bk.qattn_correct(self.layout, cache, q, lens, self.idx if self.k > 0 else None, self.k, self.ws,
                             self.out, stream)
            return self.out
        bk.kv_pack_append(self.layout, cache, k_new, v_new, 1, pos, stream)
        return self.attend(cache, q, lens, stream)


class HybridPipeline:
    """The hybrid step (JetFire README, introduction: a low-bit cache on the
    GPU, the high-precision correction of the top-k tokens on the host) over
    several layers, the host's exact pass overlapped with GPU work.

    A layer's query depends on the previous layer's output, so the host pass
    of a layer cannot overlap the next layer's scan of the same sequences.
    The batch is split into `micro` micro-batches (contiguous batch rows)
    instead: while the host computes micro-batch m's exact states of layer i
    (qattn_exact_host), the GPU runs the other micro-batches' work -- their
    scans, and their merges and next-layer scans.  Per micro-batch and layer:
    qattn_decode_step (append of the new token, scan, top-k) and the copies of
    the rows and the query to pinned host memory, then an event; the host
    waits for that event only (no stream-wide synchronise), computes, and
    enqueues the copy of the states and qattn_correct_hybrid, then the
    micro-batch's next layer.  Every enqueue is on the current stream, so a
    micro-batch's buffers are reused only after its previous merge.
    caches[i] must keep its shadow in pinned host memory."""

    def __init__(self, layout: bk.Layout, k: int, max_len: int, micro: int = 2, device="cuda",
                 n_threads: int = 0):
        import torch
        if layout.batch % micro:
            raise ValueError("the batch must split into equal micro-batches")
        self.layout, self.k, self.micro, self.n_threads = layout, int(k), int(micro), int(n_threads)
        self.nb = layout.batch // micro
        self.steps = []
        for m in range(micro):
            lay_m = bk.make_layout(self.nb, layout.n_q_heads, layout.n_kv_heads, layout.capacity, layout.k_bits,
                                   layout.v_bits, head_dim=layout.head_dim, group=layout.group,
                                   query_bits=layout.query_bits, key_format=layout.key_format)
            st = DecodeStep(lay_m, k, max_len, device=device)
            L = lay_m
            st.h_idx = torch.empty(st.idx.numel(), dtype=torch.int32, pin_memory=True)
            st.h_q = torch.empty(L.batch * L.n_q_heads * L.head_dim, dtype=torch.float16, pin_memory=True)
            st.h_state = torch.empty(L.batch * L.n_q_heads * (L.head_dim + 2), dtype=torch.float32,
                                     pin_memory=True)
            st.d_state = torch.empty_like(st.h_state, device=st.out.device)
            self.steps.append(st)

    def run(self, caches, qs, k_news, v_news, pos, outs=None):
        """Layer i appends (k_news[i], v_news[i]) at pos[b] and attends over
        pos[b] + 1 tokens of caches[i] with qs[i] ([B][Hq][D] fp16, device),
        its output into outs[i] ([B*Hq*D] fp32, device; one buffer reused
        for every layer when outs is None).  The schedule runs natively
        (qattn_hybrid_layers); returns outs."""
        import torch
        nl = len(caches)
        if outs is None:
            L = self.layout
            if not hasattr(self, "_out"):
                self._out = torch.empty(L.batch * L.n_q_heads * L.head_dim, dtype=torch.float32,
                                        device=self.steps[0].out.device)
            outs = [self._out] * nl
        slots = [dict(sigma=st.sigma, idx=st.idx, ws=st.ws, state_dev=st.d_state, idx_host=st.h_idx,
                      q_host=st.h_q, state_host=st.h_state) for st in self.steps]
        bk.qattn_hybrid_layers(self.layout, list(caches), list(qs), list(k_news), list(v_news), pos, self.k,
                               self.micro, slots, list(outs), self.n_threads)
        return outs
