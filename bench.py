#!/usr/bin/env python3
"""Benchmark of the block-sparse tiled attention hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input that is
already resident in HBM: the fused token-to-tile layout of Q, K, V and the gate
(bsa_tile_layout, one launch) followed by the block-sparse attention forward
(bsa_fwd, one launch).  The reported value is effective TFLOP/s counting only
the valid tokens of the selected tiles (4*D*vbs[i]*vbs[j] per listed pair).

Prints one JSON line.  Default workload: the dense-limit shape (B=1, H=6,
D=128, 31200 tokens in 244 tiles of 128, the last of 96; every query tile
lists every key tile), the largest configuration and the one the 50 % target
is set on.  --workload picks another.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "effective TFLOPS (selected tiles only) + % bf16 MFMA peak, ms/call"
WORKLOAD_NAMES = {
    "ragged": "tile128_ragged_25pct",
    "dense": "dense_limit_31200",
    "video": "video_sparse_64tile",
    "stress": "stress_ragged_naninf",
    "dense25": "dense_shape_25pct",
    "dense256": "dense_limit_31200_tile256",
    "video_cube": "video_cube_64tile",
    "tiny": "tiny",
}
KERNEL_SOURCES = ["bsa_fwd_common.h", "bsa_fwd.hip"]


def pair_flops(w):
    """Valid-token FLOPs of one attention pass: sum of 4*D*vbs[i]*vbs[j] over listed pairs."""
    live = np.arange(w.MS)[None, None, None, :] < w.q2k_num[..., None]
    kv = np.where(live, w.vbs[w.q2k_idx], 0).sum(-1)  # [B, H, NT] valid keys per item
    return int(4 * w.D * (kv * w.vbs[None, None, :]).sum()), kv


def full_tile_flops(w):
    live = np.arange(w.MS)[None, None, None, :] < w.q2k_num[..., None]
    return int(4 * w.D * w.T * w.T * live.sum())


def kernel_source_digest():
    """sha256 (first 16 hex digits) of the forward kernel's sources with comments and
    whitespace removed: a change to the code, not to its comments, makes the committed
    traffic counters stale."""
    import re

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_tiled_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None  # the kernel changed since the counters were taken
    return rec.get("fwd_bytes_per_launch")


def library_source_digest():
    """sha256 (first 16 hex digits) of every library source and the header: the revision
    of the code that was timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_tiled_amd", "csrc")
    for path in sorted(os.path.join(csrc, n) for n in os.listdir(csrc)) + \
            [os.path.join(ROOT, "include", "bsa.h")]:
        if path.endswith((".hip", ".h")):
            with open(path, "rb") as f:
                h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def clock_levels():
    """The shader (sclk) and memory (mclk) clock levels the driver exposes, in MHz, with the
    one current when read ("*"); None where sysfs does not show them."""
    import glob

    out = {}
    for kind in ("sclk", "mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}")):
            try:
                with open(path) as f:
                    lines = [ln.strip() for ln in f if ln.strip()]
            except OSError:
                continue
            if lines:
                out[kind] = lines
                break
    return out or None


def run_env(dev):
    """The device and software the numbers were taken on."""
    import torch

    props = torch.cuda.get_device_properties(dev)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"device": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm,
            "torch": torch.__version__, "hip": torch.version.hip,
            "library_source_sha256": library_source_digest(), "clock_levels_mhz": clock_levels()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(w, kv, budget_flops, threads=None, seconds=10.0):
    """Time the CPU oracle (as is) on a bounded sample of the workload's rows: whole
    non-empty query tiles in a seeded random order up to ``budget_flops``, repeated
    until about ``seconds`` of wall time (at most three times that)."""
    import oracle

    items = np.argwhere(kv > 0)  # (b, h, i) with keys
    rng = np.random.default_rng(0)
    rng.shuffle(items)
    rows, flops = [], 0
    for b, h, i in items:
        vq = int(w.vbs[i])
        f = 4 * w.D * int(kv[b, h, i]) * vq
        if flops and flops + f > budget_flops:
            break
        base = (b * w.H + h) * w.S + i * w.T
        rows.extend(range(base, base + vq))
        flops += f
    rows = np.array(rows, np.int64)
    threads = cpu_threads() if threads is None else threads
    passes, dt = 0, 0.0
    while dt < seconds and (passes == 0 or dt * (passes + 1) / passes < 3 * seconds):
        t0 = time.perf_counter()
        oracle.fwd_rows(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs, w.T, rows, nthreads=threads)
        dt += time.perf_counter() - t0
        passes += 1
    n_items = len(set((r // w.T) for r in rows))
    return {
        "value": flops * passes / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_items} of {int((kv > 0).sum())} non-empty query tiles ({rows.size} valid "
                  f"rows, {flops / 1e9:.2f} GFLOP) of the same workload, fp32 C oracle, "
                  f"{passes} passes in {dt:.1f} s",
        "seconds": round(dt, 2),
    }


def cpu_protocol(bench_name, bench_w, bench_kv):
    """The oracle timed on every configuration: all host threads on each (a bounded
    sample, about 3 s), and one thread on the tiny and ragged configurations."""
    from block_sparse_tiled_amd import inputs as gen

    res = {"all_threads": {}, "single_thread": {}}
    for name in ("tiny", "ragged", "video", "dense", "stress"):
        if name == bench_name:
            w, kv = bench_w, bench_kv
        else:
            w = gen.make(name)
            kv = pair_flops(w)[1]
        print(f"[bench] CPU oracle on {name}", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, kv, 8e9, seconds=3.0)
        res["all_threads"][WORKLOAD_NAMES[name]] = {k: cb[k] for k in ("value", "cores", "sample")}
        if name in ("tiny", "ragged"):
            cb1 = cpu_baseline(w, kv, 1e9, threads=1, seconds=3.0)
            res["single_thread"][WORKLOAD_NAMES[name]] = {k: cb1[k] for k in ("value", "sample")}
        del w, kv
    return res


def run_backward(args, w, flops_fwd, put, dev):
    """One training pass of the attention: bsa_fwd_lse, bsa_bwd_k2q and bsa_bwd, inputs
    resident in HBM.  Algorithmic backward FLOPs: the five products of the plain
    backward (S recomputed, dP, dV, dQ, dK), 2.5 times the forward's valid-token count."""
    import torch

    import block_sparse_tiled_amd as bsa

    q, k, v = put(w.q), put(w.k), put(w.v)
    idx, num, vbs = put(w.q2k_idx), put(w.q2k_num), put(w.vbs)
    rng = np.random.default_rng(17)
    from block_sparse_tiled_amd import inputs as gen

    dout = put(gen.to_bf16_bits(rng.standard_normal(w.q.shape).astype(np.float32)))
    out, out_lo = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream(dev)
    ws_bytes = bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bsa.fwd_lse(q, k, v, idx, num, vbs, w.T, out=out, lse=lse, out_lo=out_lo, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        k2q_idx, k2q_num = bsa.bwd_k2q(idx, num)
        if ev is not None:
            ev[2].record(stream)
        bsa.bwd(q, k, v, out, out_lo, dout, lse, idx, num, k2q_idx, k2q_num, vbs, w.T, dq=dq, dk=dk,
                dv=dv)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(events[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = lambda a, b: float(np.mean([e[a].elapsed_time(e[b]) for e in events]))  # noqa: E731
    fwd_ms, k2q_ms, bwd_ms = ms(0, 1), ms(1, 2), ms(2, 3)
    flops_bwd = int(2.5 * flops_fwd)
    ms_step = wall * 1e3 / args.steps
    rec = {
        "metric": "backward effective TFLOPS (selected tiles only) + % bf16 MFMA peak, ms/call",
        "value": round(flops_bwd / (bwd_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "B": w.B, "H": w.H, "D": w.D,
                   "tile": w.T, "num_tiles": w.NT, "max_sel": w.MS,
                   "flops_bwd_valid_tokens": flops_bwd,
                   "step": "bsa_fwd_lse + bsa_bwd_k2q + bsa_bwd (delta, dQ, dK/dV kernels)"},
        "fwd_lse_ms": round(fwd_ms, 5),
        "k2q_ms": round(k2q_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "train_pass_tflops": round((flops_fwd + flops_bwd) / (ms_step * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "bsa_bwd (delta + dq_kernel + dkv_kernel)",
                     "achieved": round(flops_bwd / (bwd_ms * 1e-3) / 1e12, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(rec), flush=True)


def run_coarse(args, w, put, dev):
    """The coarse stage (bsa_coarse: pooling, coarse logits, top-k selection, coarse output)
    on the workload's tiled Q, K, V, keeping as many tiles per query tile as the workload's
    lists hold.  Prints its own JSON line.  The roofline kernel is the pooling, which reads
    every valid row of Q, K and V once (HBM-bound); its algorithmic bytes are divided by the
    whole stage's time (four launches), a lower bound on that kernel's own rate."""
    import torch

    import block_sparse_tiled_amd as bsa

    q, k, v, vbs = put(w.q), put(w.k), put(w.v), put(w.vbs)
    topk = int(w.MS)
    idx = torch.empty((w.B, w.H, w.NT, topk), dtype=torch.int32, device=dev)
    num = torch.empty((w.B, w.H, w.NT), dtype=torch.int32, device=dev)
    oc = torch.empty((w.B, w.H, w.NT, w.D), dtype=torch.float32, device=dev)
    ws = torch.empty(bsa.coarse_workspace_size(w.B, w.H, w.NT, w.T, w.D), dtype=torch.uint8,
                     device=dev)

    def call():
        bsa.coarse(q, k, v, vbs, w.T, topk, q2k_idx=idx, q2k_num=num, coarse_out=oc, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        call()
        ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    # The whole layer, from token-major Q, K, V and gate to the token-major output, in
    # its two orders: layout of the four tensors, coarse stage, fine attention on the
    # coarse stage's lists, combine, way back; against the layout that also pools,
    # the coarse stage from the pooled tiles, the fine attention, and the combine done
    # in the way back.  (And the first two steps of each, on their own.)
    tok = [put(w.tok[x]) for x in ("q", "k", "v", "gate")]
    src_map = put(w.tile_src_token)
    src_np = np.asarray(w.tile_src_token)
    token_row_np = np.full(w.tok["q"].shape[1], -1, np.int32)
    token_row_np[src_np[src_np >= 0]] = np.nonzero(src_np >= 0)[0]
    token_row = put(token_row_np)
    tiled = [torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev) for _ in tok]
    pooled = torch.empty((3, w.B, w.H, w.NT, w.D), dtype=torch.float32, device=dev)
    fine = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev)
    layer_out = torch.empty(tuple(w.tok["q"].shape), dtype=torch.bfloat16, device=dev)
    fws = bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, topk)
    fwd_ws = torch.empty(fws, dtype=torch.uint8, device=dev) if fws else None

    def separate_head():
        bsa.tile_layout(tok, src_map, w.T, outs=tiled)
        bsa.coarse(tiled[0], tiled[1], tiled[2], vbs, w.T, topk, q2k_idx=idx, q2k_num=num,
                   coarse_out=oc, workspace=ws)

    def fused_head():
        bsa.tile_layout_pool(tok, src_map, vbs, w.T, outs=tiled, pooled=pooled)
        bsa.coarse_pooled(pooled, vbs, w.T, topk, q2k_idx=idx, q2k_num=num, coarse_out=oc,
                          workspace=ws)

    def separate_layer():
        separate_head()
        bsa.fwd(tiled[0], tiled[1], tiled[2], idx, num, vbs, w.T, out=fine, workspace=fwd_ws)
        bsa.coarse_combine(fine, tiled[3], oc, vbs, w.T)
        bsa.tile_unlayout([fine], token_row, w.T, outs=[layer_out])

    def fused_layer():
        fused_head()
        bsa.fwd(tiled[0], tiled[1], tiled[2], idx, num, vbs, w.T, out=fine, workspace=fwd_ws)
        bsa.tile_unlayout_combine(fine, tiled[3], oc, vbs, token_row, w.T, dst=layer_out)

    layer_ms = {}
    for name, fn in (("layout_then_coarse_ms", separate_head),
                     ("layout_pool_then_coarse_pooled_ms", fused_head),
                     ("layer_ms", separate_layer), ("layer_fused_ms", fused_layer)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evl = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for s in range(args.steps):
            evl[s][0].record()
            fn()
            evl[s][1].record()
        torch.cuda.synchronize()
        layer_ms[name] = round(float(np.mean([e[0].elapsed_time(e[1]) for e in evl])), 5)

    valid = int(w.vbs.sum())
    pool_bytes = 3 * w.B * w.H * valid * w.D * 2 + 3 * w.B * w.H * w.NT * w.D * 4
    logit_flops = 2 * w.B * w.H * w.NT * w.NT * w.D
    rec = {
        "metric": "coarse stage ms/call (pooling, logits, top-k selection, coarse output)",
        "value": round(ms, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": False,
        "dtype": "f32 (bf16 inputs)",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "B": w.B, "H": w.H, "D": w.D,
                   "tile": w.T, "num_tiles": w.NT, "topk": topk, "valid_tokens": valid,
                   "pool_bytes": pool_bytes, "logit_flops": logit_flops,
                   "step": "bsa_coarse (4 launches), inputs resident in HBM"},
        "roofline": {"bound": "hbm", "kernel": "coarse_pool_kernel (whole stage time)",
                     "achieved": round(pool_bytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(pool_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": None},
        "layer_orders": layer_ms,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-gflop", type=float, default=80.0,
                    help="size of the row sample the CPU oracle is timed on")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB copy kernel (HBM counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the training pass instead: log-sum-exp forward, transposed lists, "
                         "backward (prints its own JSON line)")
    ap.add_argument("--cold", type=int, default=0,
                    help="also time this many forward calls, each after a 1 GiB scratch write "
                         "(cache-cold; off by default so that profiles count only the timed steps)")
    ap.add_argument("--coarse", action="store_true",
                    help="time the coarse stage (tile selection and coarse output) instead "
                         "(prints its own JSON line)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time only the attention launch (the tile buffers are laid out once "
                         "before timing) -- for profiling")
    ap.add_argument("--cpu-protocol", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the oracle on every configuration (all threads; one thread "
                         "on tiny and ragged)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by batch*head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_tiled_amd as bsa
    from block_sparse_tiled_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = gen.make(args.workload, gate=True)
    flops, kv = pair_flops(w)

    def put(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    if args.backward:
        run_backward(args, w, flops, put, dev)
        return
    if args.coarse:
        run_coarse(args, w, put, dev)
        return

    tok = [put(w.tok[x]) for x in ("q", "k", "v", "gate")]
    src_map = put(w.tile_src_token)
    idx, num, vbs = put(w.q2k_idx), put(w.q2k_num), put(w.vbs)
    tiled = [torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev) for _ in tok]
    out = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws_bytes = bsa.workspace_size(w.B, w.H, w.NT, w.T, w.D, w.MS)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    if args.fwd_only:  # the forward always reads the laid-out inputs, never uninitialised memory
        bsa.tile_layout(tok, src_map, w.T, outs=tiled)

    def step(ev=None):
        if not args.fwd_only:
            if ev is not None:
                ev[0].record(stream)
            bsa.tile_layout(tok, src_map, w.T, outs=tiled)
        if ev is not None:
            ev[1].record(stream)
        bsa.fwd(tiled[0], tiled[1], tiled[2], idx, num, vbs, w.T, out=out, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    fwd_ms = [events[s][1].elapsed_time(events[s][2]) for s in range(args.steps)]
    lay_ms = ([events[s][0].elapsed_time(events[s][1]) for s in range(args.steps)]
              if not args.fwd_only else [0.0])
    fwd_avg = float(np.mean(fwd_ms))
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (fwd_avg * 1e-3) / 1e12
    traffic = load_traffic(args.workload)

    layout_bytes = 4 * 2 * w.D * (w.B * w.H) * (int(w.vbs.sum()) + w.S)

    # The way back (not part of the step): the attention output gathered from the
    # tile buffer to token-major order through the token -> tile-row map.
    src_np = np.asarray(w.tile_src_token, np.int64)
    tokens = int((src_np >= 0).sum())
    token_row = np.zeros(tokens, np.int32)
    token_row[src_np[src_np >= 0]] = np.flatnonzero(src_np >= 0)
    row_dev = put(token_row)
    back = [torch.empty((w.B, tokens, w.H, w.D), dtype=torch.bfloat16, device=dev)]
    for _ in range(3):
        bsa.tile_unlayout([out], row_dev, w.T, outs=back)
    un_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n_un = 20
    torch.cuda.synchronize()
    un_ev[0].record(stream)
    for _ in range(n_un):
        bsa.tile_unlayout([out], row_dev, w.T, outs=back)
    un_ev[1].record(stream)
    torch.cuda.synchronize()
    unlayout_ms = un_ev[0].elapsed_time(un_ev[1]) / n_un
    unlayout_bytes = 2 * 2 * w.D * w.B * w.H * tokens + 4 * tokens

    cold_ms = None
    if args.cold > 0:
        # forward calls after a 1 GiB scratch write each, which evicts L2 and MALL
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.cold)]
        for c in range(args.cold):
            scratch.fill_(float(c))
            cold_ev[c][0].record(stream)
            bsa.fwd(tiled[0], tiled[1], tiled[2], idx, num, vbs, w.T, out=out, workspace=ws)
            cold_ev[c][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in cold_ev]))
        del scratch
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload],
            "B": w.B, "H": w.H, "D": w.D, "tile": w.T, "num_tiles": w.NT, "max_sel": w.MS,
            "valid_tokens": int(w.vbs.sum()),
            "flops_valid_tokens": flops,
            "flops_full_tiles": full_tile_flops(w),
            "step": "bsa_fwd only (tile buffers laid out once before timing)" if args.fwd_only
                    else "bsa_tile_layout(q,k,v,gate) + bsa_fwd, inputs resident in HBM",
            "workspace_bytes": ws_bytes,
        },
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_avg, 5),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 5),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 5),
        "fwd_ms_cold": round(cold_ms, 5) if cold_ms is not None else None,
        "layout_ms": round(float(np.mean(lay_ms)), 5),
        "layout_gbs": (round(layout_bytes / (float(np.mean(lay_ms)) * 1e-3) / 1e9, 1)
                       if not args.fwd_only else None),
        "unlayout": {
            "kernel": "tile_unlayout_kernel",
            "what": "attention output, tile buffer -> token-major (timed apart from the step)",
            "ms": round(unlayout_ms, 5),
            "gbs": round(unlayout_bytes / (unlayout_ms * 1e-3) / 1e9, 1),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "bsa_fwd_kernel",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "kernel_source_digest": kernel_source_digest(),
        "env": run_env(dev),
    }
    if args.calibrate_copy:
        # a plain elementwise copy of known size: reads and writes 1 GiB once
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        rec["calibration_copy_bytes"] = src.numel() * 4
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        try:
            cb = cpu_baseline(w, kv, args.cpu_budget_gflop * 1e9)
            cb["value"] = round(cb["value"], 6)
            cb["cpu_model"] = cpu_model()
            if args.cpu_protocol:
                del tok, tiled, out, ws
                cb["protocol"] = cpu_protocol(args.workload, w, kv)
        except Exception as e:  # the GPU figures stand on their own; say why the baseline is missing
            print(f"[bench] CPU baseline failed: {e!r}", file=sys.stderr, flush=True)
            cb = {"value": None, "unit": "TFLOP/s", "kind": "oracle", "error": repr(e),
                  "cpu_model": cpu_model()}
        rec["cpu_baseline"] = cb
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
