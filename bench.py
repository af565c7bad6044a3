#!/usr/bin/env python
"""Throughput of shifted sparse attention (S²-Attn) forward + backward on one
MI355X, in useful TFLOP/s.

Workload: one Llama-2-7B-shaped attention layer, B=1, N=32768, H=32,
D=128, group G=8192 (ratio 1/4, shift 4096), original wrapped-roll
boundary; seeded synthetic bf16 N(0,1) q, k, v, dO resident in HBM before
the timed region.  A step is one forward (O fp32, LSE) plus one backward
(delta preprocess, then dQ/dK/dV).  Useful FLOPs count 4*D per allowed
causal pair for the forward and 10*D for the backward.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded
on the stream the library launches on (torch's current stream).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

WORKLOAD = dict(config=3, B=1, N=32768, H=32, D=128, G=8192, boundary=0,
                L=32768)
# CPU-baseline sample: every query row of one head of each class (fwd+bwd),
# i.e. 2 of the 32 heads
CPU_SAMPLE_ROWS = 32768


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line, time the ratio sweep "
                         "B=2 N=12288 H=32 D=128 for every G with shift 0 and "
                         "shift G/2 under each boundary variant (one JSON line "
                         "per entry)")
    ap.add_argument("--rope", action="store_true",
                    help="instead of the headline line, time the RoPE "
                         "prologue (rotate q and k, bf16) and its gradient "
                         "map (dq and dk, fp32, in place) at the headline "
                         "shape (one JSON line, HBM roofline)")
    ap.add_argument("--docs", type=int, default=0, metavar="MEAN_LEN",
                    help="instead of the headline line, time the headline "
                         "step under a document mask of packed samples with "
                         "geometric lengths of this mean (one JSON line; "
                         "useful work counts only same-document pairs)")
    ap.add_argument("--shard", type=int, default=0, metavar="P",
                    help="time one slice of the headline sequence cut into "
                         "P slices (sequence parallelism, halo exchange "
                         "not included)")
    ap.add_argument("--config", type=int, default=0, choices=(0, 2, 4, 5),
                    help="instead of the headline line, time another "
                         "workload (2: 8K forward, 4: ratio sweep, 5: ragged "
                         "100K): forward and both backwards, raw and "
                         "effective throughput, the oracle on a sample")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="time the backward whose dQ kernel recomputes S "
                         "and dP (s2attn_bwd) instead of the one that "
                         "stores dS (s2attn_bwd_ds, the default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device (a plain copy "
                         "kernel of known size, to calibrate HBM counters)")
    return ap.parse_args()


def code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed: two
    sources that differ only in comments or layout compile to the same
    kernels."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(read=None) -> str:
    """Hash of the kernel sources' code (see code_tokens); ``read(name)``
    returns a file's text (default: the working tree)."""
    csrc = os.path.join(ROOT, "sparse_attention_long_attn_amd", "csrc")
    if read is None:
        def read(name):
            return open(os.path.join(csrc, name)).read()
        names = os.listdir(csrc)
    else:
        names = read(None)
    h = hashlib.sha256()
    for f in sorted(names):
        if f.endswith((".hip", ".h")):
            h.update(code_tokens(read(f)).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 PMC
    summary, or None if there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def host_info():
    """Cores this process may run on, the CPU model and the BLAS backend
    numpy calls (with its thread count)."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads")
                break
    except Exception:  # pragma: no cover - informational only
        pass
    return {"cores": cores, "cpu_model": model, "blas": blas,
            "blas_threads": threads}


def oracle_run(fn, flops, sample):
    """Time one oracle call; report it as a cpu_baseline record."""
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    info = host_info()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": info["cores"], "kind": "oracle", "seconds": round(dt, 3),
            "cpu_model": info["cpu_model"], "blas": info["blas"],
            "blas_threads": info["blas_threads"], "sample": sample}


def cpu_baseline(cfg):
    """Time the float64 oracle on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    import synthetic as syn
    B, N, H, D, G = cfg["B"], cfg["N"], cfg["H"], cfg["D"], cfg["G"]
    heads = [0, H // 2]                       # one head of each class
    R = CPU_SAMPLE_ROWS
    ins = syn.make_inputs(cfg["config"], 0, B, N, H, D, with_do=True,
                          L=cfg["L"])
    x = [syn.bf16_bits_to_f64(ins[t][:, :, heads, :])
         for t in ("q", "k", "v", "do")]
    rows = np.arange(R)
    # allowed pairs of rows [0, R) in each of the two heads
    pairs = sum(int(oracle.adjacency_block(c, rows, N, G, G // 2,
                                           cfg["boundary"], cfg["L"]).sum())
                for c in (0, 1))
    return oracle_run(
        lambda: oracle.backward(*x, G, G // 2, cfg["boundary"], cfg["L"],
                                1.0 / D ** 0.5, rows=rows),
        14 * D * pairs * B,
        f"float64 oracle fwd+bwd of query rows [0,{R}) of heads {heads} "
        f"(one per head class), B={B} N={N} D={D} G={G} wrap: {pairs} "
        f"allowed pairs")


SWEEP_GS = (12288, 6144, 3072, 2048, 1536)


def sweep(args):
    """Shift ablation over the group-ratio sweep: the same step (forward,
    preprocess, dK/dV, dQ; the stored-dS backward unless --recompute-dq)
    timed with HIP events for shift 0 (plain grouping) and shift G/2 under
    each boundary variant."""
    import torch
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    from sparse_attention_long_attn_amd import work
    B, N, H, D = 2, 12288, 32, 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ins = syn.make_inputs(4, 0, B, N, H, D, with_do=True, L=N)
    q, k, v, do = (torch.from_numpy(ins[t].view("int16")).view(torch.bfloat16)
                   .to(dev) for t in ("q", "k", "v", "do"))
    del ins
    o = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
                  for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    names = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}
    for G in SWEEP_GS:
        for shift, bnd in ((0, syn.SPLIT), (G // 2, syn.SPLIT),
                           (G // 2, syn.WRAP), (G // 2, syn.CYCLIC)):
            kw = dict(G=G, shift=shift, boundary=bnd, valid_len=N)
            ws = None if args.recompute_dq else s2a.ds_workspace(
                q, G=G, shift=shift, boundary=bnd)

            def step():
                s2a.fwd(q, k, v, o=o, lse=lse, **kw)
                s2a.bwd_preprocess(o, do, delta)
                if ws is None:
                    s2a.bwd_dkdv(q, k, v, lse, delta, do, dk, dv, **kw)
                    s2a.bwd_dq(q, k, v, lse, delta, do, dq, **kw)
                else:
                    s2a.bwd_dkdv_ds(q, k, v, lse, delta, do, dk, dv, ws, **kw)
                    s2a.bwd_dq_ds(k, ws, dq, **kw)

            for _ in range(args.warmup):
                step()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            f_fwd, f_bwd = work.useful_flops(B, N, H, D, G, shift, bnd, N)
            pairs = work.total_pairs(B, N, H, G, shift, bnd, N)
            print(json.dumps({
                "metric": "S2-Attn fwd+bwd useful TFLOP/s, ratio sweep",
                "value": round((f_fwd + f_bwd) / (ms * 1e-3) / 1e12, 2),
                "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
                "steps": args.steps, "warmup": args.warmup,
                "backward": "recomputed S, dP for dQ" if ws is None
                            else "stored dS",
                "config": {"workload": f"B={B} N={N} H={H} D={D} G={G} "
                                       f"shift={shift} {names[bnd]}",
                           "group": G, "shift": shift,
                           "boundary": names[bnd], "allowed_pairs": pairs,
                           "ratio_to_full_causal": round(
                               pairs / (B * H * N * (N + 1) / 2), 4)},
            }), flush=True)
            del ws
            torch.cuda.empty_cache()


# The other workloads (each its own JSON line, never the default):
#   2  one layer's forward at 8K, G=2048, strict-causal split boundary
#   4  the group-ratio sweep, B=2 N=12288, every G, split boundary
#   5  the ragged 100K sequence (valid 100000 of 102400), G=25600, both
#      boundary variants
CONFIG_LINES = {
    2: dict(B=1, N=8192, H=32, D=128, Gs=(2048,), bnds=(1,), L=8192,
            bwd=False),
    4: dict(B=2, N=12288, H=32, D=128, Gs=SWEEP_GS, bnds=(1,), L=12288,
            bwd=True),
    5: dict(B=1, N=102400, H=32, D=128, Gs=(25600,), bnds=(0, 1), L=100000,
            bwd=True),
}


def config_bench(args):
    """Forward (and both backwards) of one other workload, with the raw
    throughput (pairs counted over the padded length, as if every position
    were valid) next to the effective one (valid pairs only), and the
    float64 oracle timed on a stated sample of the same inputs."""
    import numpy as np
    import torch
    import oracle
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    from sparse_attention_long_attn_amd import work
    c = args.config
    cfg = CONFIG_LINES[c]
    B, N, H, D, L = (cfg[k] for k in ("B", "N", "H", "D", "L"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}
    for vi, (G, bnd) in enumerate((G, b) for G in cfg["Gs"] for b in cfg["bnds"]):
        shift = G // 2
        sc = 1.0 / D ** 0.5
        ins = syn.make_inputs(c, vi, B, N, H, D, with_do=cfg["bwd"], L=L)
        t = {k: torch.from_numpy(ins[k].view("int16")).view(torch.bfloat16)
             .to(dev) for k in ins}
        kw = dict(G=G, shift=shift, boundary=bnd, valid_len=L, scale=sc)
        o = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        fwd_ms = timed(lambda: s2a.fwd(t["q"], t["k"], t["v"], o=o, lse=lse,
                                       **kw))
        eff = work.total_pairs(B, N, H, G, shift, bnd, L)
        raw = work.total_pairs(B, N, H, G, shift, bnd, N)
        line = {"metric": "S2-Attn useful TFLOP/s, other workloads",
                "config": {"workload": f"config {c}: B={B} N={N} H={H} "
                                       f"D={D} G={G} shift={shift} "
                                       f"{names[bnd]} valid_len={L}",
                           "allowed_pairs_valid": eff,
                           "allowed_pairs_padded": raw},
                "steps": args.steps, "warmup": args.warmup,
                "fwd_ms": round(fwd_ms, 4),
                "fwd_tflops_effective": round(4 * D * eff / fwd_ms / 1e9, 2),
                "fwd_tflops_raw": round(4 * D * raw / fwd_ms / 1e9, 2)}
        if cfg["bwd"]:
            dq, dk, dv = (torch.empty_like(o) for _ in range(3))
            delta = torch.empty_like(lse)
            s2a.fwd(t["q"], t["k"], t["v"], o=o, lse=lse, **kw)
            ws = s2a.ds_workspace(t["q"], G=G, shift=shift, boundary=bnd)
            for name, fn in (
                    ("stored_ds", lambda: s2a.bwd_ds(
                        t["q"], t["k"], t["v"], o, lse, t["do"], dq=dq,
                        dk=dk, dv=dv, delta=delta, ds_ws=ws, **kw)),
                    ("recompute", lambda: s2a.bwd(
                        t["q"], t["k"], t["v"], o, lse, t["do"], dq=dq,
                        dk=dk, dv=dv, delta=delta, **kw))):
                ms = timed(fn)
                line[f"bwd_{name}_ms"] = round(ms, 4)
                line[f"step_{name}_ms"] = round(ms + fwd_ms, 4)
                line[f"step_{name}_tflops_effective"] = round(
                    14 * D * eff / (ms + fwd_ms) / 1e9, 2)
                line[f"step_{name}_tflops_raw"] = round(
                    14 * D * raw / (ms + fwd_ms) / 1e9, 2)
            line["ds_workspace_bytes"] = ws.numel()
            del ws
        # the oracle on a sample: one head of each class, batch row 0,
        # over the rows of one whole group per head (all rows when a
        # forward-only workload is small enough)
        if not args.no_cpu_baseline:
            heads = [1, H - 2]
            x = {k: syn.bf16_bits_to_f64(ins[k][:1, :, heads, :]) for k in ins}
            pairs, calls = 0, []
            for hi, h in enumerate(heads):
                cls = int(h >= H // 2)
                segs = oracle.segments(N, G, shift, bnd)[cls]
                rows = (np.arange(N) if not cfg["bwd"]
                        else np.asarray(segs[len(segs) // 2]))
                pairs += int(oracle.adjacency_block(cls, rows, N, G, shift,
                                                    bnd, L).sum())
                calls.append((hi, rows))

            def run():
                for hi, rows in calls:
                    if cfg["bwd"]:
                        oracle.backward(x["q"], x["k"], x["v"], x["do"], G,
                                        shift, bnd, L, sc, heads=[hi],
                                        rows=rows)
                    else:
                        oracle.forward(x["q"], x["k"], x["v"], G, shift, bnd,
                                       L, sc, heads=[hi], rows=rows)
            per = 14 if cfg["bwd"] else 4
            line["cpu_baseline"] = oracle_run(
                run, per * D * pairs,
                f"float64 oracle {'fwd+bwd' if cfg['bwd'] else 'fwd'} of "
                f"heads {heads} (one per class), batch row 0, "
                f"{'the rows of the middle group of each class' if cfg['bwd'] else 'all rows'}"
                f": {pairs} allowed pairs")
        print(json.dumps(line), flush=True)
        del t, ins
        torch.cuda.empty_cache()


def rope_bench(args):
    """The RoPE prologue at the headline shape: two rope launches (q, k;
    bf16 in and out) and two rope_bwd launches (dq, dk; fp32, in place),
    each timed with HIP events.  Each launch streams its tensor once, so
    the algorithmic bytes are one read and one write of it."""
    import torch
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    cfg = WORKLOAD
    B, N, H, D = (cfg[k] for k in ("B", "N", "H", "D"))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ins = syn.make_inputs(cfg["config"], 0, B, N, H, D)
    q, k = (torch.from_numpy(ins[t].view("int16")).view(torch.bfloat16)
            .to(dev) for t in ("q", "k"))
    del ins
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    g = [torch.randn((B, N, H, D), device=dev) for _ in range(2)]
    rcfg = dict(base=10000.0, pos_scale=1.0, pairing="half")

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    fwd_ms = timed(lambda: (s2a.rope(q, out=qr, **rcfg),
                            s2a.rope(k, out=kr, **rcfg))) / 2
    bwd_ms = timed(lambda: (s2a.rope_bwd(g[0], out=g[0], **rcfg),
                            s2a.rope_bwd(g[1], out=g[1], **rcfg))) / 2
    elems = B * N * H * D
    fb, bb = 2 * 2 * elems, 2 * 4 * elems      # read + write per launch
    fgbs = fb / (fwd_ms * 1e-3) / 1e9
    bgbs = bb / (bwd_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "RoPE prologue HBM throughput (rotate q or k, bf16)",
        "value": round(fgbs, 1), "unit": "GB/s", "higher_is_better": True,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_launch": round(fwd_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "s2a_rope_kernel",
                     "achieved": round(fgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(fgbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_launch": fb},
        "bwd": {"ms_per_launch": round(bwd_ms, 4), "bytes_per_launch": bb,
                "achieved_gbs": round(bgbs, 1),
                "frac": round(bgbs / PEAK_HBM_GBS, 4)},
        "config": {"workload": f"RoPE at global positions, B={B} N={N} "
                               f"H={H} D={D}, half pairing, base 1e4",
                   "dtype": "bf16 (fwd), f32 (bwd)"},
    }), flush=True)


def docs_bench(args):
    """The headline step (forward, preprocess, dK/dV, dQ) under a document
    mask: packed samples of geometric length with the given mean.  Useful
    FLOPs are 14*D per allowed same-document pair; tiles whose document IDs
    cannot meet are skipped by the kernels."""
    import torch
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    from sparse_attention_long_attn_amd import work
    cfg = WORKLOAD
    B, N, H, D, G, L, bnd = (cfg[k] for k in ("B", "N", "H", "D", "G", "L",
                                              "boundary"))
    shift = G // 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ins = syn.make_inputs(cfg["config"], 0, B, N, H, D, with_do=True, L=L)
    q, k, v, do = (torch.from_numpy(ins[t].view("int16")).view(torch.bfloat16)
                   .to(dev) for t in ("q", "k", "v", "do"))
    del ins
    doc = syn.make_doc_ids(7000 + args.docs, B, N, args.docs)
    dd = torch.from_numpy(doc).to(dev)
    o = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
                  for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    kw = dict(G=G, shift=shift, boundary=bnd, valid_len=L, doc_ids=dd)

    def step():
        s2a.fwd(q, k, v, o=o, lse=lse, **kw)
        s2a.bwd_preprocess(o, do, delta)
        s2a.bwd_dkdv(q, k, v, lse, delta, do, dk, dv, **kw)
        s2a.bwd_dq(q, k, v, lse, delta, do, dq, **kw)

    for _ in range(args.warmup):
        step()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    pairs = work.total_doc_pairs(B, N, H, G, shift, bnd, L, doc)
    dense = work.total_pairs(B, N, H, G, shift, bnd, L)
    useful = 14 * D * pairs
    print(json.dumps({
        "metric": "S2-Attn fwd+bwd useful TFLOP/s under a document mask",
        "value": round(useful / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "higher_is_better": True, "ms_per_step": round(ms, 4),
        "steps": args.steps, "warmup": args.warmup,
        "config": {"workload": f"B={B} N={N} H={H} D={D} G={G} wrap, packed "
                               f"documents of mean length {args.docs}",
                   "documents": int(doc.max()) + 1, "allowed_pairs": pairs,
                   "fraction_of_unmasked_pairs": round(pairs / dense, 4)},
    }), flush=True)


def shard_bench(args):
    """One slice of the headline sequence under sequence parallelism: the
    headline workload cut into P slices on group edges, timed for a middle
    slice (a left halo of s rows, no padding).  The halo exchange, a
    point-to-point copy between devices, is not part of the timed work."""
    import torch
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    from sparse_attention_long_attn_amd import work
    cfg = WORKLOAD
    N, H, D, G, L, bnd = (cfg[k] for k in ("N", "H", "D", "G", "L",
                                           "boundary"))
    P = args.shard
    if N % P or (N // P) % G:
        raise SystemExit(f"--shard {P}: slices of N/P rows must be whole "
                         f"groups of {G}")
    T, s = N // P, G // 2
    r = 1 if P > 1 else 0
    row0 = r * T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ins = syn.make_inputs(cfg["config"], 0, 1, N, H, D, with_do=True, L=L)
    full = {t: torch.from_numpy(ins[t].view("int16")).view(torch.bfloat16)[0]
            for t in ("q", "k", "v", "do")}
    del ins
    left0, hl, hw = s2a.shard_halo(N, row0, T, G=G, boundary=bnd,
                                   valid_len=L)
    R = 2 * s if hw else s

    def ext(x):
        e = torch.zeros((R + T, H, D), dtype=x.dtype)
        e[R:] = x[row0:row0 + T]
        if hl:
            e[R - hl:R] = x[left0:left0 + hl]
        if hw:
            e[R - 2 * s:R - 2 * s + hw] = x[:hw]
        return e.to(dev)

    q = full["q"][row0:row0 + T].contiguous().to(dev)
    do = full["do"][row0:row0 + T].contiguous().to(dev)
    kx, vx = ext(full["k"]), ext(full["v"])
    del full
    o = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    dk, dv = (torch.zeros((R + T, H, D), dtype=torch.float32, device=dev)
              for _ in range(2))
    delta = torch.empty((H, T), dtype=torch.float32, device=dev)
    kw = dict(N=N, row0=row0, G=G, boundary=bnd, valid_len=L)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def step(rec=False):
        if rec:
            ev[0].record()
        s2a.fwd_shard(q, kx, vx, o=o, lse=lse, **kw)
        if rec:
            ev[1].record()
        s2a.bwd_shard(q, kx, vx, o, lse, do, dq=dq, dk=dk, dv=dv, delta=delta,
                      **kw)
        if rec:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tf = tb = 0.0
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        tf += ev[0].elapsed_time(ev[1])
        tb += ev[1].elapsed_time(ev[2])
    tf, tb = tf / args.steps, tb / args.steps
    c0, c1 = work.shard_pairs(N, row0, T, G, s, bnd, L)
    pairs = (H // 2) * (c0 + c1)
    useful = 14 * D * pairs
    ms = tf + tb
    print(json.dumps({
        "metric": "S2-Attn fwd+bwd useful TFLOP/s of one sequence-parallel "
                  "slice (halo exchange excluded)",
        "value": round(useful / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "higher_is_better": True, "ms_per_step": round(ms, 4),
        "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
        "steps": args.steps, "warmup": args.warmup,
        "config": {"workload": f"slice {r} of {P} ({T} rows from {row0}) of "
                               f"B=1 N={N} H={H} D={D} G={G} wrap",
                   "halo_rows": hl, "allowed_pairs": pairs,
                   "fraction_of_whole": round(
                       pairs / work.total_pairs(1, N, H, G, s, bnd, L), 4)},
    }), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this engine has no multi-GPU "
              "path (heads shard with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args)
        return
    if args.rope:
        rope_bench(args)
        return
    if args.docs:
        docs_bench(args)
        return
    if args.shard:
        shard_bench(args)
        return
    if args.config:
        config_bench(args)
        return

    import torch
    import synthetic as syn
    import sparse_attention_long_attn_amd as s2a
    from sparse_attention_long_attn_amd import work

    cfg = WORKLOAD
    B, N, H, D, G, L, bnd = (cfg[k] for k in ("B", "N", "H", "D", "G", "L",
                                              "boundary"))
    shift = G // 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ins = syn.make_inputs(cfg["config"], 0, B, N, H, D, with_do=True, L=L)
    q, k, v, do = (torch.from_numpy(ins[t].view("int16")).view(torch.bfloat16)
                   .to(dev) for t in ("q", "k", "v", "do"))
    del ins
    o = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
                  for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    kw = dict(G=G, shift=shift, boundary=bnd, valid_len=L)
    # the backward stores dS (bf16, 2 bytes per allowed pair) in dK/dV and
    # forms dQ from it, unless --recompute-dq asks for the other backward
    stored = not args.recompute_dq
    ws = s2a.ds_workspace(q, G=G, shift=shift, boundary=bnd) if stored else None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        s2a.fwd(q, k, v, o=o, lse=lse, **kw)
        if ev is not None:
            ev[1].record()
        s2a.bwd_preprocess(o, do, delta)
        if ev is not None:
            ev[2].record()
        if stored:
            s2a.bwd_dkdv_ds(q, k, v, lse, delta, do, dk, dv, ws, **kw)
        else:
            s2a.bwd_dkdv(q, k, v, lse, delta, do, dk, dv, **kw)
        if ev is not None:
            ev[3].record()
        if stored:
            s2a.bwd_dq_ds(k, ws, dq, **kw)
        else:
            s2a.bwd_dq(q, k, v, lse, delta, do, dq, **kw)
        if ev is not None:
            ev[4].record()

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)            # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
           for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / K
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    pre_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    dkdv_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / K
    dq_ms = sum(e[3].elapsed_time(e[4]) for e in evs) / K

    f_fwd, f_bwd = work.useful_flops(B, N, H, D, G, shift, bnd, L)
    b_fwd, b_bwd = work.algorithmic_bytes(B, N, H, D, o_bytes=4)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    # useful work of each kernel: QK^T and PV (fwd); the backward's 10*D
    # per pair is dV, dK, dP and S in the dK/dV kernel (8*D) and dQ (2*D)
    # in the dQ kernel (which, with --recompute-dq, also recomputes S and
    # dP: not counted)
    D_pairs = f_fwd // (4 * D)
    kernels = {
        "s2a_fwd_sw_kernel": (fwd_ms, f_fwd),
        "s2a_bwd_dkdv_w64_kernel": (dkdv_ms, 8 * D * D_pairs),
        ("s2a_bwd_dq_ds_kernel" if stored else "s2a_bwd_dq_sw_kernel"):
            (dq_ms, 2 * D * D_pairs),
    }
    dom = max(kernels, key=lambda n: kernels[n][0])
    dms, dfl = kernels[dom]
    achieved = dfl / (dms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(dom),
                "avg_ms": round(dms, 4),
                "flops_per_launch": dfl}

    out = {
        "metric": "S²-Attn fwd+bwd useful TFLOP/s and % bf16 MFMA peak at "
                  "N=32K, G=8K",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 q,k,v,dO (PCG64, rounded to "
                "nearest even)",
        "config": {"workload": "S2-Attn fwd+bwd, Llama-2-7B layer shape, "
                               "B=1 N=32768 H=32 D=128 G=8192 shift=4096 "
                               "wrapped-roll boundary",
                   "global_batch": B, "seq_len": N, "heads": H,
                   "head_dim": D, "group": G, "boundary": "wrap",
                   "valid_len": L, "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "backward": "stored dS" if stored else "recomputed S, dP for dQ",
        "ds_workspace_bytes": ws.numel() if stored else 0,
        "fwd_ms": round(fwd_ms, 4),
        "bwd_preprocess_ms": round(pre_ms, 4),
        "bwd_dkdv_ms": round(dkdv_ms, 4),
        "bwd_dq_ms": round(dq_ms, 4),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / ((pre_ms + dkdv_ms + dq_ms) * 1e-3) / 1e12,
                            2),
        "useful_flops_per_step": f_fwd + f_bwd,
        "algorithmic_bytes": {"fwd": b_fwd, "bwd": b_bwd},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
