"""Seeded synthetic decode-attention inputs (no method arithmetic here).

These stand in for the workloads the pages evaluate on (LongBench v1 and
needle-in-a-haystack prompts on Llama-3.1-8B, Qwen3-30B-A3B and Llama-3.3-70B,
per the JetFire README's evaluation section); neither the datasets nor the
weights are used.  Recipe:

* numpy ``default_rng(seed)`` (PCG64); values drawn in fp64 and rounded to fp16
  (round to nearest even).
* q, K, V ~ N(0, 1).
* outlier key channels: for each KV head, ``n_outlier`` distinct channels are
  multiplied by ``outlier_scale`` for every token, appended ones included
  (mirrors the outlier-channel observation in the TailorKV review).
* planted tokens (the needle analogue): ``planted`` distinct positions per
  (batch, KV head); planted token j gets, after the outlier scaling, the key
  ``|k| * (0.9 * q_h / |q_h| + sqrt(0.19) * w)`` with h = j mod G inside the
  group, w a random unit vector orthogonal to q_h and |k| the row's own norm,
  so its cosine with q_h is 0.9.  V is never planted.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int
    kbits: int
    vbits: int
    group: int
    k: int
    planted: int
    seed: int
    n_outlier: int = 4
    outlier_scale: float = 8.0
    query_bits: int = 0  # 8: approximate scores against the INT8 query (HACK's Eq. (4))
    key_format: int = 0  # 1: MXFP4 keys, fp16 query; 2: MXFP4 keys (E8M0 scales) and MXFP4 query

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five decode-attention shapes (one attention layer, all heads).
WORKLOADS = [
    Workload("tiny_k4v4_L1024", 1, 4, 1, 128, 1024, 4, 4, 32, 16, 8, 1000),
    Workload("llama8b_k4v4_L32768", 4, 32, 8, 128, 32768, 4, 4, 32, 256, 64, 1001),
    Workload("llama8b_k3v2_L32768", 4, 32, 8, 128, 32768, 3, 2, 32, 256, 64, 1002),
    Workload("qwen30b_k3v2_L32768", 4, 32, 4, 128, 32768, 3, 2, 32, 256, 0, 1003),
    Workload("llama70b_k3v2_L131072", 4, 64, 8, 128, 131072, 3, 2, 32, 512, 256, 1004),
]
# The 8B shape with the aggressive codecs of the TailorKV review (1- and
# 2-bit keys, 2-bit values, groups of 64 channels).
CODEC_WORKLOADS = [
    Workload("llama8b_k2v2g64_L32768", 4, 32, 8, 128, 32768, 2, 2, 64, 256, 64, 1005),
    Workload("llama8b_k1v2g64_L32768", 4, 32, 8, 128, 32768, 1, 2, 64, 256, 64, 1006),
    # HACK's INT8-query scores on the 8B K4V4 cache
    Workload("llama8b_k4v4_q8_L32768", 4, 32, 8, 128, 32768, 4, 4, 32, 256, 64, 1007, query_bits=8),
    # MXFP4 keys scored against the MXFP4 query (the FP4 query-key product), 4-bit values
    Workload("llama8b_mxfp4v4_L32768", 4, 32, 8, 128, 32768, 4, 4, 32, 256, 64, 1008, key_format=2),
    # the variant: MXFP4 keys scored against the fp16 query
    Workload("llama8b_mxfp4v4_f16q_L32768", 4, 32, 8, 128, 32768, 4, 4, 32, 256, 64, 1009, key_format=1),
]
BY_NAME = {w.name: w for w in WORKLOADS + CODEC_WORKLOADS}


def _f16(x: np.ndarray) -> np.ndarray:
    return x.astype(np.float16)


@dataclass
class Inputs:
    q: np.ndarray            # [B][Hq][D] fp16
    K: np.ndarray            # [B][Hkv][L][D] fp16 (cache contents, oldest first)
    V: np.ndarray            # [B][Hkv][L][D] fp16
    outlier_ch: np.ndarray   # [Hkv][n_outlier] int
    planted_pos: np.ndarray  # [B][Hkv][planted] int (sorted)


def make_inputs(w: Workload, L: int | None = None) -> Inputs:
    """The cache of `L` tokens (default w.L) plus the query, per the recipe above."""
    L = w.L if L is None else L
    rng = np.random.default_rng(w.seed)
    q64 = rng.standard_normal((w.B, w.Hq, w.D))
    q = _f16(q64)
    outlier_ch = np.stack([rng.choice(w.D, size=w.n_outlier, replace=False)
                           for _ in range(w.Hkv)]) if w.n_outlier else np.zeros((w.Hkv, 0), int)
    K = np.empty((w.B, w.Hkv, L, w.D), dtype=np.float16)
    V = np.empty((w.B, w.Hkv, L, w.D), dtype=np.float16)
    n_pl = min(w.planted, L)
    planted = np.zeros((w.B, w.Hkv, n_pl), dtype=np.int64)
    qf = q.astype(np.float64)
    for b in range(w.B):
        for kvh in range(w.Hkv):
            k = rng.standard_normal((L, w.D))
            k[:, outlier_ch[kvh]] *= w.outlier_scale
            pos = np.sort(rng.choice(L, size=n_pl, replace=False)) if n_pl else np.zeros(0, int)
            for j, t in enumerate(pos):
                h = kvh * w.G + (j % w.G)
                qh = qf[b, h] / np.linalg.norm(qf[b, h])
                r = rng.standard_normal(w.D)
                r -= (r @ qh) * qh
                r /= np.linalg.norm(r)
                k[t] = np.linalg.norm(k[t]) * (0.9 * qh + np.sqrt(0.19) * r)
            K[b, kvh] = _f16(k)
            V[b, kvh] = _f16(rng.standard_normal((L, w.D)))
            planted[b, kvh] = pos
    return Inputs(q=q, K=K, V=V, outlier_ch=outlier_ch, planted_pos=planted)


def make_new_tokens(w: Workload, n_steps: int, outlier_ch: np.ndarray, stream: int = 1):
    """Appended tokens for `n_steps` decode steps, same law, no planting.
    Returns (k_new, v_new), each [n_steps][B][Hkv][1][D] fp16."""
    rng = np.random.default_rng([w.seed, stream])
    k = rng.standard_normal((n_steps, w.B, w.Hkv, 1, w.D))
    for kvh in range(w.Hkv):
        k[:, :, kvh, :, outlier_ch[kvh]] *= w.outlier_scale
    v = rng.standard_normal((n_steps, w.B, w.Hkv, 1, w.D))
    return _f16(k), _f16(v)
