"""Benchmark of one approximate-then-correct decode-attention step on one GPU.

A step is one pass of the whole hot path for one attention layer, all heads:
kv_pack_append (one new token per sequence) -> qattn_decode_select (the
approximate scan with the per-KV-head top-k in the same launch; or, with
--two-launch, qattn_decode_approx -> topk_select) -> qattn_correct, over the
workload's context length.  Inputs are
seeded synthetic tensors (bit_kv_attention_amd.synth), resident in HBM before
timing starts.  The timed steps rotate over several independent cache copies
(as separate layers would) so that the packed bytes read per rotation exceed
the 256 MB Infinity Cache.

Output: one JSON line (rank 0) with tokens/s = batch / step time, the packed-KV
bandwidth, per-kernel times, the roofline of the dominant kernel and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0


def packed_bytes_per_token(kbits: int, vbits: int, D: int = 128, group: int = 32) -> int:
    meta = (D // group) * 4
    return D * kbits // 8 + meta + D * vbits // 8 + meta


def scan_partial_bytes(lay, L: int) -> int:
    """Bytes of split states the scan writes: per (b, query head, split) the
    max, the denominator and D accumulators (fp32); splits as the library
    chooses them (about 256 workgroups, 256-token multiples)."""
    units = lay.batch * lay.n_kv_heads
    per = -(-units * L // 256)
    per = max(256, -(-per // 256) * 256)
    nsplit = -(-L // per)
    return lay.batch * lay.n_q_heads * nsplit * (2 + lay.head_dim) * 4


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama8b_k4v4_L32768",
                    help="workload name from bit_kv_attention_amd.synth.WORKLOADS, or 'all'")
    ap.add_argument("--shadow", choices=["hbm", "host"], default="hbm")
    ap.add_argument("--blocks", type=int, default=0, metavar="NB",
                    help="select NB whole blocks of --block tokens per KV head (topk_select_blocks) "
                         "instead of the workload's top-k tokens")
    ap.add_argument("--block", type=int, default=128)
    ap.add_argument("--exact", choices=["gpu", "host"], default="gpu",
                    help="host: the exact half of the correction on the host's cores from a pinned host "
                         "shadow (qattn_exact_host + qattn_correct_hybrid)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with kv_pack_append before the scan instead of inside its launch")
    ap.add_argument("--two-launch", action="store_true",
                    help="run the scan and the top-k as two calls (qattn_decode_approx, topk_select)")
    ap.add_argument("--window", type=int, default=0,
                    help="also correct the newest WINDOW tokens of every sequence (topk_select_window)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (3 times), the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the method shards by "
              "KV head or by context length without changing the kernels); run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return 0
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep
    from bit_kv_attention_amd.synth import BY_NAME, WORKLOADS, make_inputs, make_new_tokens

    names = [w.name for w in WORKLOADS] if args.config == "all" else [args.config]
    for name in names:
        w = BY_NAME[name]
        res = bench_one(w, args, torch, bk, DecodeStep, make_inputs, make_new_tokens)
        print(json.dumps(res), flush=True)
    return 0


def bench_one(w, args, torch, bk, DecodeStep, make_inputs, make_new_tokens):
    dev = torch.device("cuda:0")
    L = w.L
    cap = ((L + 31) // 32) * 32
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group, query_bits=w.query_bits,
                         key_format=w.key_format)
    units = w.B * w.Hkv
    ppt = packed_bytes_per_token(w.kbits, w.vbits, group=w.group)
    packed = units * L * ppt
    copies = args.copies or max(1, min(8, -(-600_000_000 // packed)))

    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(w, L=L - 1)
    knew, vnew = make_new_tokens(w, 1, inp.outlier_ch)
    Kd = torch.from_numpy(inp.K).to(dev)
    Vd = torch.from_numpy(inp.V).to(dev)
    q = torch.from_numpy(inp.q).to(dev)
    kn = torch.from_numpy(knew[0]).to(dev)
    vn = torch.from_numpy(vnew[0]).to(dev)
    caches = []
    for c in range(copies):
        cache = bk.allocate_cache(lay, device=dev, shadow_on_host=(args.shadow == "host" or args.exact == "host"))
        bk.kv_pack_append(lay, cache, Kd, Vd, L - 1, [0] * w.B)
        caches.append(cache)
    del Kd, Vd
    torch.cuda.synchronize()
    W = args.window
    NB = args.blocks
    if NB:
        st = DecodeStep(lay, NB, L, device=dev, block=args.block)
    else:
        st = DecodeStep(lay, w.k, L, device=dev, window=W, fused=not args.two_launch)
    fused = st.fused and not NB and not W
    # qattn_decode_select picks the selection inside the scan's launch where that is faster
    in_scan = fused and bk.bkv_select_in_scan(lay, L, w.k)
    hybrid = args.exact == "host"
    if hybrid and not fused:
        raise SystemExit("--exact host runs with the plain top-k step (no --blocks, --window, --two-launch)")
    # When the library would run the scan and the top-k as two launches anyway,
    # the timed loop makes the two calls itself, so the scan launch is timed alone.
    fused = in_scan
    # 1- and 2-bit keys: the unselected tokens' state from a second pass (see DecodeStep)
    exclude = st.exclude and not hybrid
    exclude_scores = exclude and not NB and not W and not args.two_launch
    # the plain step appends the new token inside the scan's launch (qattn_decode_step)
    step_launch = st.fused and not NB and not W and not exclude and not hybrid and not args.separate_append
    nthr = args.cpu_threads or 16
    pos = [L - 1] * w.B  # each step writes the newest token at slot L-1, then attends over L
    lens = [L] * w.B

    def select():
        if NB > 0:
            bk.topk_select_blocks(lay, st.sigma, lens, NB, args.block, st.idx, st.ws)
        elif W > 0:
            bk.topk_select_window(lay, st.sigma, lens, w.k, W, st.idx, st.ws)
        else:
            bk.topk_select(lay, st.sigma, lens, w.k, st.idx, st.ws)

    def step(i):
        cache = caches[i % copies]
        if step_launch:
            st.step(cache, q, kn, vn, pos)
            return
        bk.kv_pack_append(lay, cache, kn, vn, 1, pos)
        if hybrid:
            st.attend_hybrid(cache, q, lens, nthr)
        else:
            st.attend(cache, q, lens)

    print(f"[bench] {w.name}: warmup {args.warmup}, timing {args.steps} steps over {copies} copies",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: the steps, with events on the library's stream (torch's
    # current stream) around the scan launch of every SAMPLE-th step for the
    # roofline figure (an event pair costs about a microsecond of the step).
    SAMPLE = 4
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(0, args.steps, SAMPLE)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        cache = caches[i % copies]
        ev_i = sev[i // SAMPLE] if i % SAMPLE == 0 else None
        if step_launch:  # the append inside the scan's launch (with the top-k too where that is faster)
            if ev_i:
                ev_i[0].record()
            bk.qattn_decode_step(lay, cache, kn, vn, q, lens, w.k if in_scan else 0, st.sigma, st.idx, st.ws)
            if ev_i:
                ev_i[1].record()
            if not in_scan:
                select()
            bk.qattn_correct(lay, cache, q, lens, st.idx, st.row, st.ws, st.out)
            continue
        bk.kv_pack_append(lay, cache, kn, vn, 1, pos)
        ev_scan = ev_i if not exclude else None  # the dominant launch: the scan, or the second pass
        ev_rest = ev_i if exclude else None
        if ev_scan:
            ev_scan[0].record()
        if exclude_scores:  # scores and rows only, then the second pass below
            bk.qattn_score_select(lay, cache, q, lens, w.k, st.sigma, st.idx, st.ws)
        elif fused:
            bk.qattn_decode_select(lay, cache, q, lens, w.k, st.sigma, st.idx, st.ws)
        else:
            bk.qattn_decode_approx(lay, cache, q, lens, st.sigma, st.ws)
        if ev_scan:
            ev_scan[1].record()
        if not fused and not exclude_scores:
            select()
        if hybrid:
            st.attend_hybrid(cache, q, lens, nthr, select=False)
        elif exclude:
            if ev_rest:
                ev_rest[0].record()
            bk.qattn_decode_unselected(lay, cache, q, lens, st.idx, st.row, st.ws)
            if ev_rest:
                ev_rest[1].record()
            bk.qattn_correct_unselected(lay, cache, q, lens, st.idx, st.row, st.ws, st.out)
        else:
            bk.qattn_correct(lay, cache, q, lens, st.idx, st.row, st.ws, st.out)
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    scan_us_timed = 1000.0 * float(np.mean([a.elapsed_time(b) for a, b in sev]))

    # Per-call breakdown: the same steps again with events around each call.
    if hybrid:
        names = ("kv_pack_append", "qattn_decode_select", "exact_host_and_copies+qattn_correct_hybrid")
        calls = (lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, pos),
                 lambda c: bk.qattn_decode_select(lay, c, q, lens, w.k, st.sigma, st.idx, st.ws),
                 lambda c: st.attend_hybrid(c, q, lens, nthr, select=False))
    elif step_launch:
        names = ["qattn_decode_step"] + ([] if in_scan else ["topk_select"]) + ["qattn_correct"]
        calls = [lambda c: bk.qattn_decode_step(lay, c, kn, vn, q, lens, w.k if in_scan else 0, st.sigma, st.idx,
                                                st.ws)] + \
                ([] if in_scan else [lambda c: select()]) + \
                [lambda c: bk.qattn_correct(lay, c, q, lens, st.idx, st.row, st.ws, st.out)]
    else:
        if exclude_scores:
            names = ["kv_pack_append", "qattn_score_select"]
            calls = [lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, pos),
                     lambda c: bk.qattn_score_select(lay, c, q, lens, w.k, st.sigma, st.idx, st.ws)]
        elif fused:
            names = ["kv_pack_append", "qattn_decode_select"]
            calls = [lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, pos),
                     lambda c: bk.qattn_decode_select(lay, c, q, lens, w.k, st.sigma, st.idx, st.ws)]
        else:
            names = ["kv_pack_append", "qattn_decode_approx", "topk_select"]
            calls = [lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, pos),
                     lambda c: bk.qattn_decode_approx(lay, c, q, lens, st.sigma, st.ws),
                     lambda c: select()]
        if exclude:
            names += ["qattn_decode_unselected", "qattn_correct_unselected"]
            calls += [lambda c: bk.qattn_decode_unselected(lay, c, q, lens, st.idx, st.row, st.ws),
                      lambda c: bk.qattn_correct_unselected(lay, c, q, lens, st.idx, st.row, st.ws, st.out)]
        else:
            names += ["qattn_correct"]
            calls += [lambda c: bk.qattn_correct(lay, c, q, lens, st.idx, st.row, st.ws, st.out)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(args.steps)]
    for i in range(args.steps):
        cache = caches[i % copies]
        for j, call in enumerate(calls):
            ev[i][j][0].record()
            call(cache)
            ev[i][j][1].record()
    torch.cuda.synchronize()
    kus = {n: 1000.0 * float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(args.steps)]))
           for j, n in enumerate(names)}

    tokens_per_s = w.B / (ms / 1000.0)
    packed_gbps = packed / (ms / 1000.0) / 1e9
    # dominant kernel: the approximate scan.  Algorithmic bytes per launch =
    # packed codes + meta of K and V for every token of every unit, the fp32
    # selection score written per token, and the split partial states written
    # (plus, with the selection in the same launch, the k indices per unit).
    if exclude:  # the second pass: packed bytes and split states, the rows read (no sigma)
        scan_bytes = units * L * ppt + scan_partial_bytes(lay, L) + units * st.row * 4
    else:
        scan_bytes = units * L * (ppt + 4) + scan_partial_bytes(lay, L) + (units * w.k * 4 if in_scan else 0)
        if step_launch:  # + the appended rows read and the token's codes, meta and shadow rows written
            scan_bytes += units * (2 * 256 + ppt + 2 * 256)
    scan_s = scan_us_timed / 1e6
    achieved = scan_bytes / scan_s / 1e9
    traffic = measured_traffic(w.name)
    res = {
        "metric": "decode attention tokens/s + packed-KV HBM GB/s (% of peak), 32K & 128K ctx",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "n_q_heads": w.Hq, "n_kv_heads": w.Hkv,
                   "head_dim": w.D, "context": L, "k_bits": w.kbits, "v_bits": w.vbits,
                   "group": w.group, "query_bits": w.query_bits, "key_format": "mxfp4" if w.key_format else "affine", "top_k": 0 if NB else w.k,
                   "recent_window": W,
                   "blocks": NB, "block": args.block if NB else 0,
                   "shadow": "host" if hybrid else args.shadow, "exact": args.exact,
                   "cache_copies": copies,
                   "selection_in_scan_launch": bool(in_scan), "append_in_scan_launch": bool(step_launch),
                   "unselected_second_pass": bool(exclude),
                   "parallelism": "single GPU"},
        "packed_kv_GBps": round(packed_gbps, 1),
        "packed_kv_frac_of_hbm_peak": round(packed_gbps / HBM_PEAK_GBPS, 4),
        "kernel_us": {n: round(v, 2) for n, v in kus.items()},
        "wall_s_timed_region": round(t_wall, 3),
        "roofline": {"kernel": ("qattn_decode_unselected (second pass)" if exclude else
                               "qattn_decode_step (append + scan + top-k launch)" if step_launch and in_scan else
                               "qattn_decode_step (append + scan launch)" if step_launch else
                               "qattn_decode_select (scan + top-k launch)" if in_scan else
                               "qattn_decode_approx (scan launch)"), "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": scan_bytes,
                     "kernel_us_per_launch": round(scan_us_timed, 2), "launches_timed": len(sev)},
    }
    if not args.no_cpu_baseline and W == 0 and NB == 0 and not hybrid:  # the oracle's timed path has no window
        res["cpu_baseline"] = cpu_baseline(w, inp, knew, vnew, args.cpu_threads)
    del caches
    torch.cuda.empty_cache()
    return res


SCAN_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_kv_attention_amd", "csrc",
                           "decode_approx.hip")
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def measured_traffic(workload):
    """HBM bytes per launch of the scan kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by what the same
    counter reads for a plain copy of known size), or None when there is no
    summary for this workload or the kernel source has changed since the
    counters were taken."""
    import hashlib
    path = os.path.join(PROFILES, f"decode_approx_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    with open(SCAN_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if vals.get("source_sha256") != sha or "hbm_bytes_per_launch" not in vals:
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def cpu_baseline(w, inp, knew, vnew, threads):
    """The oracle, as it stands, on a bounded sample of the same step: `threads`
    (batch, KV head) units, one thread each; the full step would take
    units/threads times as long."""
    import oracle
    oracle.build(force=False)
    threads = threads or min(16, os.cpu_count() or 1)
    units = w.B * w.Hkv
    sample = min(threads, units)
    oracle.set_threads(sample)
    L = w.L
    cap = ((L + 31) // 32) * 32
    sel = [(u // w.Hkv, u % w.Hkv) for u in range(sample)]
    s = oracle.Shape(1, w.G * sample, sample, 128, w.kbits, w.vbits, w.group, cap, w.key_format)
    # fold the sampled units into one batch row of `sample` KV heads
    K = np.stack([inp.K[b, h] for b, h in sel])[None]
    V = np.stack([inp.V[b, h] for b, h in sel])[None]
    q = np.concatenate([inp.q[b, h * w.G:(h + 1) * w.G] for b, h in sel])[None]
    kn = np.stack([knew[0][b, h] for b, h in sel])[None]
    vn = np.stack([vnew[0][b, h] for b, h in sel])[None]
    cache = oracle.Cache(s)
    cache.append(K, V, np.zeros(1, np.int32))
    t = time.perf_counter()
    cache.append(kn, vn, np.array([L - 1], np.int32))
    cache.decode(q, np.array([L], np.int32), w.k, qbits=w.query_bits)
    dt = time.perf_counter() - t
    t_step = dt * units / sample
    return {"value": round(w.B / t_step, 4), "unit": "tokens/s", "cores": sample, "kind": "oracle",
            "sample": f"{sample} of {units} (batch, KV head) units of one step at context {L} "
                      f"(append + approximate scores + top-{w.k} + corrected output), one thread "
                      f"per unit; {dt:.2f} s measured, scaled by {units}/{sample}"}


if __name__ == "__main__":
    sys.exit(main())
