"""Benchmark of one approximate-then-correct decode-attention step on one GPU.

A step is one pass of the whole hot path for one attention layer, all heads:
the append of one new token per sequence, the approximate scan over the
packed cache, the per-KV-head top-k and the exact correction, over the
workload's context length.  It runs either as one launch
(qattn_decode_fused) or as separate launches (qattn_decode_step, topk_select
when the selection is not in the scan's launch, qattn_correct); by default
both are timed during warm-up and the faster one is the step timed.

Inputs are seeded synthetic tensors (bit_kv_attention_amd.synth), resident in
HBM before timing starts.  The timed steps rotate over several independent
cache copies (as separate layers would) so that the packed bytes read per
rotation exceed the 256 MB Infinity Cache.

Output: one JSON line with tokens/s = batch / step time on the 32K workload,
the packed-KV bandwidth and its fraction of HBM peak, per-launch times, the
roofline of the dominant kernel, the CPU oracle on the host's cores, and the
same figures for the 128K context (and its pinned-host-shadow variant) under
"contexts".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
HOST_THREADS = 16  # the host-core share of one GPU on the GPU machines
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "bit_kv_attention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def packed_bytes_per_token(kbits: int, vbits: int, D: int = 128, group: int = 32, key_format: int = 0) -> int:
    """Codes plus fp16 scale and zero of K and V, per token and KV head (key
    format 2: one E8M0 byte per 32 key channels in place of the key meta)."""
    meta = (D // group) * 4
    kmeta = D // 32 if key_format == 2 else meta
    return D * kbits // 8 + kmeta + D * vbits // 8 + meta


def bench_layers(w, args, torch) -> int:
    """N layers per step, each with a cache of its own (the same tokens):
    per-layer time of (a) the all-GPU step (the fused launch where it runs),
    (b) the hybrid step run layer after layer (attend_hybrid: one wait per
    layer for the rows, host pass, merge), and (c) the hybrid step pipelined
    over two micro-batches (HybridPipeline: the host pass of one micro-batch
    overlaps the other's GPU work).  Wall clock around `steps` steps after
    `warmup`; one JSON line."""
    from bit_kv_attention_amd import binding as bk
    from bit_kv_attention_amd.step import DecodeStep, HybridPipeline
    from bit_kv_attention_amd.synth import make_inputs, make_new_tokens
    dev = torch.device("cuda:0")
    nl, L = args.layers, w.L
    cap = ((L + 31) // 32) * 32
    lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group, query_bits=w.query_bits,
                         key_format=w.key_format)
    log(f"{w.name}: {nl} layers: generating inputs")
    inp = make_inputs(w, L=L - 1)
    knew, vnew = make_new_tokens(w, 1, inp.outlier_ch)
    Kd, Vd = torch.from_numpy(inp.K).to(dev), torch.from_numpy(inp.V).to(dev)
    q = torch.from_numpy(inp.q).to(dev)
    kn, vn = torch.from_numpy(knew[0]).to(dev), torch.from_numpy(vnew[0]).to(dev)
    pos = [L - 1] * w.B
    dev_caches, host_caches = [], []
    for _ in range(nl):
        for lst, on_host in ((dev_caches, False), (host_caches, True)):
            c = bk.allocate_cache(lay, device=dev, shadow_on_host=on_host)
            bk.kv_pack_append(lay, c, Kd, Vd, L - 1, [0] * w.B)
            lst.append(c)
    del Kd, Vd
    torch.cuda.synchronize()
    gpu_steps = [DecodeStep(lay, w.k, L, device=dev, one_launch=True) for _ in range(nl)]
    hyb_steps = [DecodeStep(lay, w.k, L, device=dev, one_launch=False) for _ in range(nl)]
    pipe = HybridPipeline(lay, w.k, L, micro=2, device=dev, n_threads=args.cpu_threads)
    lens = [L] * w.B

    def gpu_step():
        for i in range(nl):
            gpu_steps[i].step(dev_caches[i], q, kn, vn, pos)

    def serial_step():
        for i in range(nl):
            st = hyb_steps[i]
            bk.qattn_decode_step(lay, host_caches[i], kn, vn, q, lens, w.k, st.sigma, st.idx, st.ws)
            st.attend_hybrid(host_caches[i], q, lens, args.cpu_threads, select=False)

    def pipe_step():
        pipe.run(host_caches, [q] * nl, [kn] * nl, [vn] * nl, pos)

    res = {}
    for name, fn in (("exact_gpu", gpu_step), ("exact_host_serial", serial_step), ("exact_host_pipelined", pipe_step)):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t) * 1e6 / args.steps / nl
        res[name + "_us_per_layer"] = round(us, 2)
        log(f"{w.name}: {name}: {us:.2f} µs per layer")
    units = w.B * w.Hkv
    kk = min(w.k, L)
    pcie = units * w.k * 4 + w.B * w.Hq * w.D * 2 + w.B * w.Hq * (w.D + 2) * 4 + units * 2 * w.D * 2
    host_read = units * kk * 2 * w.D * 2
    t_pipe = res["exact_host_pipelined_us_per_layer"]
    print(json.dumps({"mode": "layers", "config": {"workload": w.name, "layers": nl, "micro_batches": 2,
                                                   "host_threads": args.cpu_threads},
                      **res,
                      "pcie_bytes_per_layer": pcie,
                      "pcie_GBps_at_pipelined_rate": round(pcie / t_pipe / 1e3, 2),
                      "pcie_peak_GBps": 64.0,
                      "host_shadow_read_bytes_per_layer": host_read,
                      "host_read_GBps_at_pipelined_rate": round(host_read / t_pipe / 1e3, 2),
                      "host_cores": os.cpu_count()}), flush=True)
    return 0


def read_ceiling(nbytes: int, torch, copies: int = 1) -> int:
    """The plain streaming read (probe/read_ceiling.hip) of nbytes, 20 timed
    launches per grid size after 3 untimed ones, rotating over `copies`
    buffers (several copies whose total exceeds the 256 MB last-level cache
    keep a buffer of the scan's size from being served by it); prints one
    JSON line with GB/s per grid and the best."""
    import ctypes as C
    lib = C.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_kv_attention_amd",
                              "libbkvprobe.so"))
    lib.bkv_probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    nbytes -= nbytes % 16
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    out = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    turn = [0]
    for grid in (256, 512, 1024, 2048, 4096, 8192):
        def go():
            buf = bufs[turn[0] % copies]
            turn[0] += 1
            st = lib.bkv_probe_read(buf.data_ptr(), nbytes, out.data_ptr(), grid, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"bkv_probe_read: hipError {st}")
        for _ in range(3):
            go()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            go()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        res[str(grid)] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1)}
        log(f"read ceiling: {nbytes} B, grid {grid}: {us:.2f} µs, {nbytes / us / 1e3:.1f} GB/s")
    best = max(v["GBps"] for v in res.values())
    print(json.dumps({"read_ceiling_bytes": nbytes, "copies": copies, "grids": res, "best_GBps": best,
                      "best_frac_of_8000": round(best / 8000.0, 4)}), flush=True)
    return 0


def num_splits(units: int, L: int) -> int:
    """The library's split count (about 256 workgroups, 256-token multiples)."""
    per = -(-units * L // 256)
    per = max(256, -(-per // 256) * 256)
    return -(-L // per)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama8b_k4v4_L32768",
                    help="workload of the headline line (bit_kv_attention_amd.synth.BY_NAME)")
    ap.add_argument("--contexts", default="llama70b_k3v2_L131072",
                    help="comma-separated workloads reported under 'contexts' ('none' for none)")
    ap.add_argument("--no-host-shadow", action="store_true",
                    help="skip the pinned-host-shadow variant of the context workloads")
    ap.add_argument("--path", choices=["auto", "fused", "separate"], default="auto",
                    help="fused: qattn_decode_fused; separate: the separate launches; auto: the faster")
    ap.add_argument("--runs", type=int, default=3, help="runs of the protocol figure (median reported)")
    ap.add_argument("--protocol-steps", type=int, default=128)
    ap.add_argument("--shadow", choices=["hbm", "host"], default="hbm")
    ap.add_argument("--blocks", type=int, default=0, metavar="NB",
                    help="select NB whole blocks of --block tokens per KV head (topk_select_blocks)")
    ap.add_argument("--block", type=int, default=128)
    ap.add_argument("--exact", choices=["gpu", "host"], default="gpu",
                    help="host: the exact half of the correction on the host's cores (qattn_exact_host)")
    ap.add_argument("--window", type=int, default=0,
                    help="also correct the newest WINDOW tokens of every sequence (topk_select_window)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=HOST_THREADS)
    ap.add_argument("--layers", type=int, default=0, metavar="N",
                    help="only time N layers per step (each its own cache): the all-GPU step, the hybrid "
                         "step per layer, and the hybrid step pipelined over two micro-batches")
    ap.add_argument("--read-ceiling", type=int, default=0, metavar="BYTES",
                    help="only time a plain streaming read of BYTES bytes (bit_kv_attention_amd/probe), "
                         "the practical HBM read ceiling, over several grid sizes")
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

    if args.read_ceiling:
        return read_ceiling(args.read_ceiling, torch, max(args.copies, 1))
    if args.layers:
        from bit_kv_attention_amd.synth import BY_NAME
        return bench_layers(BY_NAME[args.config], args, torch)

    from bit_kv_attention_amd.synth import BY_NAME
    res = bench_one(BY_NAME[args.config], args, torch, shadow=args.shadow)
    ctx = {}
    plain = not (args.blocks or args.window or args.exact == "host")
    for name in [c for c in args.contexts.split(",") if c and c != "none"]:
        if name == args.config:
            continue
        ctx[name] = bench_one(BY_NAME[name], args, torch, shadow="hbm", line=False)
        if plain and not args.no_host_shadow:
            ctx[name + "_host_shadow"] = bench_one(BY_NAME[name], args, torch, shadow="host", line=False)
    if ctx:
        res["contexts"] = ctx
    print(json.dumps(res), flush=True)
    return 0


class Workbench:
    """Caches, buffers and the calls of one workload's step."""

    def __init__(self, w, args, torch, shadow):
        from bit_kv_attention_amd import binding as bk
        from bit_kv_attention_amd.step import DecodeStep
        from bit_kv_attention_amd.synth import make_inputs, make_new_tokens
        self.bk, self.torch, self.w, self.args = bk, torch, w, args
        dev = torch.device("cuda:0")
        L = w.L
        cap = ((L + 31) // 32) * 32
        self.lay = lay = bk.make_layout(w.B, w.Hq, w.Hkv, cap, w.kbits, w.vbits, group=w.group,
                                        query_bits=w.query_bits, key_format=w.key_format)
        self.units = w.B * w.Hkv
        self.ppt = packed_bytes_per_token(w.kbits, w.vbits, group=w.group, key_format=w.key_format)
        self.packed = self.units * L * self.ppt
        self.copies = args.copies or max(1, min(8, -(-600_000_000 // self.packed)))
        self.host_shadow = shadow == "host" or args.exact == "host"
        log(f"{w.name}: generating inputs")
        self.inp = make_inputs(w, L=L - 1)
        self.knew, self.vnew = make_new_tokens(w, 1, self.inp.outlier_ch)
        Kd = torch.from_numpy(self.inp.K).to(dev)
        Vd = torch.from_numpy(self.inp.V).to(dev)
        self.q = torch.from_numpy(self.inp.q).to(dev)
        self.kn = torch.from_numpy(self.knew[0]).to(dev)
        self.vn = torch.from_numpy(self.vnew[0]).to(dev)
        self.caches = []
        for _ in range(self.copies):
            cache = bk.allocate_cache(lay, device=dev, shadow_on_host=self.host_shadow)
            bk.kv_pack_append(lay, cache, Kd, Vd, L - 1, [0] * w.B)
            self.caches.append(cache)
        del Kd, Vd
        torch.cuda.synchronize()
        self.NB, self.W = args.blocks, args.window
        if self.NB:
            self.st = DecodeStep(lay, self.NB, L, device=dev, block=args.block)
        else:
            self.st = DecodeStep(lay, w.k, L, device=dev, window=self.W, one_launch=False)
        self.pos = [L - 1] * w.B  # each step writes the newest token at slot L-1, then attends over L
        self.lens = [L] * w.B
        self.plain = not (self.NB or self.W or args.exact == "host" or self.st.exclude)
        self.fused_ok = self.plain and bk.bkv_fused_supported(lay, L, w.k)
        self.in_scan = bk.bkv_select_in_scan(lay, L, w.k)

    # ---- the step's calls, per path; each entry is (name, call(cache)) --------
    def calls(self, path):
        bk, st, lay, w, q, kn, vn, lens = self.bk, self.st, self.lay, self.w, self.q, self.kn, self.vn, self.lens
        if path == "fused":
            return [("qattn_decode_fused",
                     lambda c: bk.qattn_decode_fused(lay, c, kn, vn, q, lens, w.k, st.sigma, st.idx, st.out, st.ws))]
        if self.args.exact == "host":
            return [("kv_pack_append", lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, self.pos)),
                    ("qattn_decode_select",
                     lambda c: bk.qattn_decode_select(lay, c, q, lens, w.k, st.sigma, st.idx, st.ws)),
                    ("exact_host_and_copies+qattn_correct_hybrid",
                     lambda c: st.attend_hybrid(c, q, lens, self.args.cpu_threads, select=False))]
        if st.exclude:  # 1- and 2-bit keys: scores and rows, then a pass over the unselected tokens
            return [("kv_pack_append", lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, self.pos)),
                    ("qattn_score_select",
                     lambda c: bk.qattn_score_select(lay, c, q, lens, w.k, st.sigma, st.idx, st.ws)),
                    ("qattn_decode_unselected",
                     lambda c: bk.qattn_decode_unselected(lay, c, q, lens, st.idx, st.row, st.ws)),
                    ("qattn_correct_unselected",
                     lambda c: bk.qattn_correct_unselected(lay, c, q, lens, st.idx, st.row, st.ws, st.out))]
        if self.NB or self.W:
            def select(c):
                if self.NB:
                    bk.topk_select_blocks(lay, st.sigma, lens, self.NB, self.args.block, st.idx, st.ws)
                else:
                    bk.topk_select_window(lay, st.sigma, lens, w.k, self.W, st.idx, st.ws)
            if self.NB:  # block rows: the correction over contiguous tiles
                correct = ("qattn_correct_blocks",
                           lambda c: bk.qattn_correct_blocks(lay, c, q, lens, st.idx, self.NB, self.args.block, st.ws,
                                                             st.out))
            else:
                correct = ("qattn_correct",
                           lambda c: bk.qattn_correct(lay, c, q, lens, st.idx, st.row, st.ws, st.out))
            return [("kv_pack_append", lambda c: bk.kv_pack_append(lay, c, kn, vn, 1, self.pos)),
                    ("qattn_decode_approx", lambda c: bk.qattn_decode_approx(lay, c, q, lens, st.sigma, st.ws)),
                    ("topk_select_blocks" if self.NB else "topk_select_window", select), correct]
        out = [("qattn_decode_step",
                lambda c: bk.qattn_decode_step(lay, c, kn, vn, q, lens, w.k if self.in_scan else 0, st.sigma,
                                               st.idx, st.ws))]
        if not self.in_scan:
            out.append(("topk_select", lambda c: bk.topk_select(lay, st.sigma, lens, w.k, st.idx, st.ws)))
        out.append(("qattn_correct", lambda c: bk.qattn_correct(lay, c, q, lens, st.idx, st.row, st.ws, st.out)))
        return out

    def run_steps(self, calls, n, start=0):
        for i in range(n):
            c = self.caches[(start + i) % self.copies]
            for _, f in calls:
                f(c)

    def time_steps(self, calls, n, start=0):
        """ms per step over n steps (events on the library's stream = torch's current stream)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        self.run_steps(calls, n, start)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def per_call_us(self, calls, n):
        """Mean µs of every call, with events around each launch."""
        torch = self.torch
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
              for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            c = self.caches[i % self.copies]
            for j, (_, f) in enumerate(calls):
                ev[i][j][0].record()
                f(c)
                ev[i][j][1].record()
        torch.cuda.synchronize()
        return {name: 1000.0 * float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(n)]))
                for j, (name, _) in enumerate(calls)}


# The sources the scan kernel (and the fused step, which is its FUSE build) is
# compiled from: decode_approx.hip and every header it includes.
SCAN_SOURCES = ("decode_approx.hip", "bkv_internal.h", "fused_tail.h", "correct_lane.h", "quant_lane.h",
                "select_lds.h")


def kernel_sources_sha256() -> str:
    """One hash over the scan kernel's sources (and the public header): a
    counter summary of the scan or the fused step holds for the kernels built
    from exactly these sources."""
    h = hashlib.sha256()
    for name in SCAN_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "bitkv.h"), "rb") as f:
        h.update(b"bitkv.h\0" + f.read())
    return h.hexdigest()


def profile_summary(kernel: str, workload: str):
    """The committed counter and duration summary of `kernel` on `workload`
    (profiles/<kernel>_<workload>_traffic.txt: HBM bytes per launch from
    FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for a
    plain copy of known size, and the kernel's median rocprof duration), or
    None when there is none or the kernel sources have changed since it was
    taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return vals


def bench_one(w, args, torch, shadow="hbm", line=True):
    wb = Workbench(w, args, torch, shadow)
    units, L, copies = wb.units, w.L, wb.copies
    # ---- the path: both timed after warm-up, the faster one kept --------------------
    paths = {}
    cand = [args.path] if args.path != "auto" else ["separate", "fused"]
    for p in cand:
        if p == "fused" and not wb.fused_ok:
            continue
        calls = wb.calls(p)
        wb.run_steps(calls, max(args.warmup, 1))
        paths[p] = round(1000.0 * wb.time_steps(calls, 20), 2)
    if not paths:
        raise SystemExit(f"no runnable path for {w.name} (--path {args.path})")
    path = min(paths, key=paths.get)
    calls = wb.calls(path)
    log(f"{w.name} [{shadow} shadow]: path {path} (warm-up µs/step {paths}); timing {args.steps} steps "
        f"over {copies} copies")

    # ---- the timed region: exactly `steps` steps ---------------------------------
    wb.run_steps(calls, args.warmup)
    t_wall = time.perf_counter()
    ms = wb.time_steps(calls, args.steps)
    t_wall = time.perf_counter() - t_wall
    # the protocol figure: median over runs of protocol-steps steps each
    run_ms = [wb.time_steps(calls, args.protocol_steps) for _ in range(args.runs)]
    # per-launch durations (events around each launch), for the roofline
    kus = wb.per_call_us(calls, max(args.steps, 20))

    tokens_per_s = w.B / (ms / 1000.0)
    packed_gbps = wb.packed / (ms / 1000.0) / 1e9
    # dominant kernel and its algorithmic bytes per launch
    nsplit = num_splits(units, L)
    states = w.B * w.Hq * nsplit * (2 + w.D) * 4  # split records written (and read back once)
    append_bytes = units * (2 * 256 + wb.ppt + 2 * 256)  # the new rows read; codes, meta, shadow written
    if path == "fused":
        kname = "qattn_decode_fused"
        shadow_bytes = units * w.k * 2 * 256  # the selected tokens' exact K and V rows
        extended = wb.packed + units * L * 4 + 2 * states + shadow_bytes + append_bytes + w.B * w.Hq * w.D * 4
    elif wb.st.exclude:
        kname = "qattn_decode_unselected"
        extended = wb.packed + states + units * wb.st.row * 4
    else:
        kname = "qattn_decode_step" if "qattn_decode_step" in kus else "qattn_decode_approx"
        extended = wb.packed + units * L * 4 + states + (units * w.k * 4 if wb.in_scan else 0)
        if kname == "qattn_decode_step":
            extended += append_bytes
    k_us = kus[kname]
    achieved = wb.packed / (k_us / 1e6) / 1e9
    prof = None if wb.host_shadow else profile_summary(kname, w.name)
    traffic = int(float(prof["hbm_bytes_per_launch"])) if prof and "hbm_bytes_per_launch" in prof else None
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
                   "group": w.group, "query_bits": w.query_bits,
                   "key_format": {0: "affine", 1: "mxfp4_fp16_query", 2: "mxfp4_fp4_query"}.get(
                       w.key_format, str(w.key_format)),
                   "top_k": 0 if wb.NB else w.k, "recent_window": wb.W,
                   "blocks": wb.NB, "block": args.block if wb.NB else 0,
                   "shadow": "host" if wb.host_shadow else "hbm", "exact": args.exact,
                   "cache_copies": copies, "path": path, "parallelism": "single GPU"},
        "packed_kv_GBps": round(packed_gbps, 1),
        "packed_kv_frac_of_hbm_peak": round(packed_gbps / HBM_PEAK_GBPS, 4),
        "path_warmup_us_per_step": paths,
        "protocol": {"runs": args.runs, "steps_per_run": args.protocol_steps,
                     "median_ms_per_step": round(float(np.median(run_ms)), 5),
                     "run_ms_per_step": [round(x, 5) for x in run_ms],
                     "median_tokens_per_s": round(w.B / (float(np.median(run_ms)) / 1000.0), 1)},
        "kernel_us": {n: round(v, 2) for n, v in kus.items()},
        "wall_s_timed_region": round(t_wall, 3),
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": wb.packed, "bytes_basis": "packed K/V codes + meta",
                     "extended_bytes_per_launch": int(extended),
                     "extended_frac": round(extended / (k_us / 1e6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "kernel_us_per_launch": round(k_us, 2),
                     "timing": "HIP events around each launch (they include the launch's dispatch latency)"},
    }
    if path == "fused" and "separate" in paths:
        # the fused launch holds the whole step (scan, selection, correction,
        # merge); beside it, the separate launches' calls on the same step
        # (events around each call; a call may hold several launches)
        sk = wb.per_call_us(wb.calls("separate"), max(args.steps, 20))
        res["separate_path"] = {"ms_per_step": round(paths["separate"] / 1000.0, 5),
                                "us_per_call": {n: round(v, 2) for n, v in sk.items()}}
    if prof and "rocprof_median_us" in prof:  # the committed kernel-trace figure beside the live one
        r_us = float(prof["rocprof_median_us"])
        res["roofline"]["rocprof_kernel_us_median"] = r_us
        res["roofline"]["rocprof_frac"] = round(wb.packed / (r_us / 1e6) / 1e9 / HBM_PEAK_GBPS, 4)
    if wb.host_shadow:
        # the selected rows cross PCIe: per step units * k * (K + V) * 256 B
        pcie = units * w.k * 2 * 256
        res["pcie_bytes_per_step"] = pcie
        res["pcie_GBps_if_correction_bound"] = round(pcie / (ms / 1000.0) / 1e9, 2)
    if not line:
        for key in ("metric", "unit", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
                    "dtype", "data"):
            res.pop(key)
    if not args.no_cpu_baseline and not wb.host_shadow and not (wb.NB or wb.W):
        res["cpu_baseline"] = cpu_baseline(wb, args)
    del wb
    torch.cuda.empty_cache()
    return res


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def cpu_baseline(wb, args):
    """The oracle, as it stands, on the same step: the append of the new token
    and the decode of every (batch, KV head) unit of the workload (OpenMP over
    the units on the host-core share of one GPU), plus the same for one unit
    on one thread.  The whole step, not a sample."""
    import oracle
    oracle.build(force=False)
    w = wb.w
    L = w.L
    cap = ((L + 31) // 32) * 32
    model, ncpu = cpu_info()
    threads = min(args.cpu_threads, ncpu)
    log(f"{w.name}: cpu oracle on {threads} threads")
    s = oracle.Shape(w.B, w.Hq, w.Hkv, 128, w.kbits, w.vbits, w.group, cap, w.key_format)
    cache = oracle.Cache(s)
    cache.append(wb.inp.K, wb.inp.V, np.zeros(w.B, np.int32))
    oracle.set_threads(threads)
    runs = 3 if L <= 32768 else 1
    times = []
    for r in range(runs):
        t = time.perf_counter()
        cache.append(wb.knew[0], wb.vnew[0], np.full(w.B, L - 1, np.int32))
        cache.decode(wb.inp.q, np.full(w.B, L, np.int32), w.k, qbits=w.query_bits)
        times.append(time.perf_counter() - t)
    t_step = float(np.median(times))
    # one unit on one thread
    s1 = oracle.Shape(1, w.G, 1, 128, w.kbits, w.vbits, w.group, cap, w.key_format)
    c1 = oracle.Cache(s1)
    c1.append(wb.inp.K[:1, :1], wb.inp.V[:1, :1], np.zeros(1, np.int32))
    oracle.set_threads(1)
    t = time.perf_counter()
    c1.append(wb.knew[0][:1, :1], wb.vnew[0][:1, :1], np.array([L - 1], np.int32))
    c1.decode(np.ascontiguousarray(wb.inp.q[:1, :w.G]), np.array([L], np.int32), w.k, qbits=w.query_bits)
    t1 = time.perf_counter() - t
    return {"value": round(w.B / t_step, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole step: all {wb.units} (batch, KV head) units at context {L} (append + "
                      f"approximate scores + top-{w.k} + corrected output), OpenMP over units, median of "
                      f"{runs} run(s)",
            "threads": threads, "host_cores": ncpu, "cpu_model": model,
            "step_s": round(t_step, 3), "run_s": [round(x, 3) for x in times],
            "single_thread_s_per_unit": round(t1, 3),
            "single_thread_step_s_estimate": round(t1 * wb.units, 2),
            "packed_GBps": round(wb.packed / t_step / 1e9, 4)}


if __name__ == "__main__":
    sys.exit(main())
