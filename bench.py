#!/usr/bin/env python3
"""Throughput of exact attention forward + backward on one MI355X.

One step = fa_forward followed by the two backward stages (dQ, which also
forms D = rowsum(dO * O), then dK/dV -- exactly what fa_backward enqueues)
over one batch of synthetic input already resident in device memory.  Default workload: the
GPT-2-medium attention shape (B 64, H 16, N 1024, d 64, bfloat16, causal,
scale 1/8).

Credited FLOPs: forward 4*B*H*N^2*d (halved when causal), backward 2.5x the
forward.  Per-kernel durations come from HIP events recorded on the stream
the kernels run on; the roofline object reports the dominant kernel's
algorithmic work per launch divided by its average duration.  The CPU
baseline times the fp64 oracle (S and P materialised) on a bounded sample of
the same workload on this host's cores.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one
GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "attention fwd+bwd TFLOP/s & % bf16 MFMA peak (B64 H16 N1024 d64 causal)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic.json"
KERNELS = ("fwd", "bwd_dq", "bwd_dkdv")
DROPOUT_SEED = 0x5EED0F00D


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_medium")
    ap.add_argument("--fwd-only", action="store_true", help="time only the forward kernel")
    ap.add_argument("--mask", choices=("none", "band", "band_global"), default="none",
                    help="block-sparse attention through fa_forward_sparse / fa_backward_sparse "
                         "with a 128x128 tile mask: 'band' = tiles within two of the diagonal, "
                         "'band_global' = the band plus tile row 0 and tile column 0 (the first "
                         "128 positions as global tokens)")
    ap.add_argument("--balanced", action="store_true",
                    help="with --mask: run fa_forward_sparse_balanced / "
                         "fa_backward_sparse_balanced over a schedule built from the mask")
    ap.add_argument("--seg", type=int, default=0,
                    help="with --balanced: most tiles per work item (0 = the library's default)")
    ap.add_argument("--splits", type=int, default=1,
                    help="forward through fa_forward_split with this many key ranges "
                         "(implies --fwd-only when > 1)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="drop probability of the fused dropout (fa_forward_dropout / "
                         "fa_backward_dropout); 0 = no dropout")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward (fa_forward_fp8) on inputs quantised beforehand "
                         "with fa_quantize_fp8; implies --fwd-only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-big-d", action="store_true",
                    help="skip the head-dim-256 forward that the default run times beside the "
                         "headline step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args(argv)


# Translation unit of each timed kernel: its source file and the headers it includes.
KERNEL_SOURCES = {
    "fwd": ("fa_fwd.hip", "fa_device.h", "fa_dropout.h", "fa_launch.h"),
    "bwd_dq": ("fa_bwd.hip", "fa_device.h", "fa_dropout.h", "fa_launch.h"),
    "bwd_dkdv": ("fa_bwd.hip", "fa_device.h", "fa_dropout.h", "fa_launch.h"),
    "bwd_pre": ("fa_bwd.hip", "fa_device.h", "fa_dropout.h", "fa_launch.h"),
}


def source_digest(kernel: str) -> str:
    """sha256 over the sources a kernel is compiled from (counters go stale when they change)."""
    h = hashlib.sha256()
    csrc = ROOT / "exact_io_aware_09_amd" / "csrc"
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        h.update((csrc / name).read_bytes())
    return h.hexdigest()


def visible_pairs(w) -> int:
    """(query, key) pairs that contribute, over all heads."""
    per_head = w.N * (w.N + 1) // 2 if w.causal else w.N * w.N
    return w.B * w.H * per_head


def band_mask(N):
    """Tile mask of a sliding window: tiles with |I - J| <= 2 (int32, CPU).

    Every tile row and column holds at most five set tiles, so the work of
    the workgroups (one per tile row in the forward and dQ kernels, one per
    tile column in the dK/dV kernel) stays balanced.
    """
    import torch

    nb = (N + 127) // 128
    i = torch.arange(nb)
    return ((i.unsqueeze(1) - i.unsqueeze(0)).abs() <= 2).to(torch.int32)


def tile_mask(kind, N):
    """'band', or 'band_global': the band plus a global first tile row and column,
    whose whole work falls on one workgroup per head unless it is split."""
    m = band_mask(N)
    if kind == "band_global":
        m[0, :] = 1
        m[:, 0] = 1
    return m


MASK_NAMES = {"band": "band |I-J|<=2", "band_global": "band |I-J|<=2 + global tile row/column 0"}


def mask_pairs(w, mask) -> int:
    """Visible (query, key) pairs of a tile mask, over all heads."""
    import torch

    N = w.N
    sizes = torch.tensor([min(128, N - 128 * t) for t in range(mask.shape[0])], dtype=torch.int64)
    full = (mask.to(torch.int64) * sizes.unsqueeze(1) * sizes.unsqueeze(0))
    if w.causal:
        # diagonal tiles keep their lower triangle only; tiles above it vanish
        tri = torch.tril(torch.ones_like(full))
        diag = torch.diag(torch.diagonal(mask).to(torch.int64) * sizes * (sizes + 1) // 2)
        full = full * tri - torch.diag(torch.diag(full)) + diag
    return int(full.sum()) * w.B * w.H


def credited_flops(w):
    fwd = 4 * w.B * w.H * w.N * w.N * w.d
    if w.causal:
        fwd //= 2
    return fwd, fwd * 5 // 2


def algorithmic(w, kernel, elem_bytes):
    """(bound, amount per launch, unit) for each kernel.

    Matrix-core work counts 2*d FLOPs per visible (query, key) pair per
    contraction: forward 2 (Q K^T, P V), dK/dV 4 (Q K^T, dO V^T, P^T dO,
    dS^T Q), dQ 3 (Q K^T, dO V^T, dS K).  The standalone D preprocess (not
    part of a step) is a streaming pass: it reads O and dO once and writes
    one float per row.
    """
    e = elem_bytes
    pairs = visible_pairs(w)
    if kernel in ("fwd", "fwd_split"):  # fwd_split: partial kernel + merge, timed together
        return "mfma", 2 * 2 * w.d * pairs, "FLOP"
    if kernel == "bwd_dkdv":
        return "mfma", 4 * 2 * w.d * pairs, "FLOP"
    if kernel == "bwd_dq":
        return "mfma", 3 * 2 * w.d * pairs, "FLOP"
    rows = w.B * w.H * w.N
    return "hbm", 2 * rows * w.d * e + 4 * rows, "B"


def stored_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counters, if still valid."""
    try:
        data = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    if data.get("workload") != workload or kernel not in KERNEL_SOURCES:
        return None
    k = data.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != source_digest(kernel):
        return None
    return int(k["fetch_bytes"]) + int(k["write_bytes"])


def host_cpu() -> str:
    """CPU model of the host (first 'model name' of /proc/cpuinfo)."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def blas_library() -> str:
    """BLAS torch's CPU matrix products call, from torch's build configuration."""
    import re

    import torch

    m = re.search(r"BLAS_INFO=([^,\s]+)", torch.__config__.show())
    return m.group(1) if m else "unknown"


def cpu_fields(threads_used: int):
    """Host description reported beside the CPU baseline."""
    return {"cores": host_cores(), "threads": threads_used, "blas": blas_library(),
            "cpu_model": host_cpu()}


def cpu_baseline_sampled(w, seconds: float):
    """Time the sampled-row oracle on query rows of the first head (N too large for S)."""
    import torch

    from exact_io_aware_09_amd.workloads import sample_rows, workload_inputs
    from oracle import sampled as SM

    q, k, v, do = (t[0, 0].clone() for t in workload_inputs(w))
    qi, _ = sample_rows(w.seed, 0, 0, w.H, w.N)
    done, t_used, chunk = 0, 0.0, 16
    while t_used < seconds and done < len(qi):
        rows = torch.as_tensor(qi[done:done + chunk])
        t0 = time.perf_counter()
        SM.query_rows(q, k, v, do, rows, w.scale, w.causal)
        t_used += time.perf_counter() - t0
        done += len(rows)
    # credited FLOPs of those rows: forward 4d per visible pair, backward 2.5x
    pairs = sum((int(r) + 1) if w.causal else w.N for r in qi[:done])
    tflops = 4 * w.d * pairs * 3.5 / t_used / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        **cpu_fields(torch.get_num_threads()),
        "kind": "oracle",
        "sample": (f"fp64 sampled-row oracle (full score rows, O, LSE and dQ per row) on {done} "
                   f"query rows of head 0 of the {w.name} workload (N={w.N}, d={w.d}, "
                   f"causal={w.causal}); {t_used:.1f} s; credited FLOPs of those rows / time; "
                   "sampled, not comparable with the full-tensor baselines"),
    }


def cpu_baseline(w, seconds: float):
    """Time the fp64 oracle on the first heads of the same workload."""
    import torch

    from exact_io_aware_09_amd.workloads import make_inputs
    from oracle import attention as A  # the baseline is the oracle itself

    if w.sampled:
        return cpu_baseline_sampled(w, seconds)

    # the workload's own inputs (same seed), flattened to heads
    q, k, v, do = (t.reshape(w.B * w.H, w.N, w.d) for t in make_inputs(w.shape, w.dtype, w.seed, w.mult))
    heads_done, t_used = 0, 0.0
    chunk = 8
    while t_used < seconds and heads_done < w.B * w.H:
        sl = slice(heads_done, min(w.B * w.H, heads_done + chunk))
        t0 = time.perf_counter()
        A.per_head(A.attention_forward_backward, (q[sl], k[sl], v[sl], do[sl]),
                   w.scale, w.causal, heads_per_chunk=chunk)
        t_used += time.perf_counter() - t0
        heads_done += sl.stop - sl.start
    fwd, bwd = credited_flops(w)
    per_head = (fwd + bwd) / (w.B * w.H)
    tflops = per_head * heads_done / t_used / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        **cpu_fields(torch.get_num_threads()),
        "kind": "oracle",
        "sample": (f"fp64 oracle forward+backward (S, P materialised) on {heads_done} heads "
                   f"(N={w.N}, d={w.d}, causal={w.causal}) of the {w.name} workload's "
                   f"{w.B * w.H}; {t_used:.1f} s; credited FLOPs of those heads / time"),
    }


def big_d_forward(steps: int = 10, warmup: int = 2):
    """Forward throughput at head dim 256, long sequence (B 2, H 16, N 16384, d 256).

    The second throughput target beside the headline step: fa_forward alone on
    the workload's own seeded inputs, timed with HIP events on the launch
    stream; credited FLOPs 4*B*H*N^2*d (non-causal).
    """
    import torch

    from exact_io_aware_09_amd import _lib
    from exact_io_aware_09_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS["big_d"]
    B, H, N, d = w.shape
    dev = torch.device("cuda:0")
    q, k, v, _ = (t.to(dev) for t in make_inputs(w.shape, w.dtype, w.seed, w.mult))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = [t.data_ptr() for t in (q, k, v, o, lse)]

    def run():
        rc = _lib.fa_forward(*P, B, H, N, d, w.scale, int(w.causal), _lib.FA_BF16, stream.cuda_stream)
        if rc != _lib.FA_OK:
            raise _lib.FAError(rc, "fa_forward")

    for _ in range(warmup):
        run()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    ms = sum(ts) / steps
    flops = 4 * B * H * N * N * d
    tflops = flops / (ms * 1e-3) / 1e12
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
            "steps": steps, "ms": round(ms, 4), "ms_median": round(ts[len(ts) // 2], 4),
            "tflops": round(tflops, 2), "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2)}


def calibrate_copy():
    import torch

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "launches": 3}), flush=True)


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the attention kernels run on one "
              "GPU's share of heads); --gpus must be 1.", file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy()
        return 0

    import exact_io_aware_09_amd as fa
    from exact_io_aware_09_amd import _lib
    from exact_io_aware_09_amd.workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    if args.splits > 1:
        args.fwd_only = True
    dtype_name = "bf16" if w.dtype == torch.bfloat16 else "f32"
    dt = _lib.FA_BF16 if dtype_name == "bf16" else _lib.FA_F32
    dev = torch.device("cuda:0")
    B, H, N, d = w.shape

    q, k, v, do = (t.to(dev) for t in workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    sparse = args.mask != "none"
    drop = args.dropout > 0.0
    if drop and (sparse or args.splits > 1):
        print("bench.py: --dropout runs the dense path only", file=sys.stderr)
        return 2
    if args.fp8 and (drop or sparse or args.splits > 1 or dtype_name != "bf16"):
        print("bench.py: --fp8 runs the dense bfloat16-input path only", file=sys.stderr)
        return 2
    if args.fp8:
        args.fwd_only = True
        q8, qs = fa.quantize_fp8(q)
        k8, ks = fa.quantize_fp8(k)
        v8, vs = fa.quantize_fp8(v, keys=True)
        P8 = [t.data_ptr() for t in (q8, qs, k8, ks, v8, vs)]
    if args.balanced and not sparse:
        print("bench.py: --balanced needs --mask", file=sys.stderr)
        return 2
    fused = sparse or drop  # one backward call: events around forward and backward only
    maskc = tile_mask(args.mask, N) if sparse else None
    maskd = maskc.to(dev) if sparse else None
    wsb = fa.workspace_bytes(B, H, N, d, w.dtype)
    sched = None
    if args.balanced:
        sched = fa.sparse_schedule(maskc, N, w.causal, B, H, seg_tiles=args.seg).to(dev)
        sh, sdv = sched.host.ctypes.data, sched.device_copy.data_ptr()
        wsb = max(wsb, _lib.fa_sparse_workspace_bytes(sh, B, H, N, d, 0),
                  _lib.fa_sparse_workspace_bytes(sh, B, H, N, d, 1))
    if args.splits > 1:
        wsb = max(wsb, _lib.fa_forward_split_workspace_bytes(B, H, N, d, args.splits, dt))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = [t.data_ptr() for t in (q, k, v, o, lse, do, dq, dk, dv, ws)]

    def call(rc, name):
        if rc != _lib.FA_OK:
            raise fa.FAError(rc, name)

    def launches(ev=None):
        """One step; if `ev` is given, record events between the kernels."""
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        if sched is not None:
            call(_lib.fa_forward_sparse_balanced(P[0], P[1], P[2], P[3], P[4], sh, sdv, P[9], wsb,
                                                 B, H, N, d, w.scale, int(w.causal), dt, sp),
                 "fa_forward_sparse_balanced")
            rec(1)
            if args.fwd_only:
                return
            call(_lib.fa_backward_sparse_balanced(P[0], P[1], P[2], P[3], P[5], P[4], sh, sdv,
                                                  P[6], P[7], P[8], P[9], wsb, B, H, N, d,
                                                  w.scale, int(w.causal), dt, sp),
                 "fa_backward_sparse_balanced")
            rec(2)
            return
        if sparse:
            call(_lib.fa_forward_sparse(P[0], P[1], P[2], P[3], P[4], maskd.data_ptr(), B, H, N,
                                        d, w.scale, int(w.causal), dt, sp), "fa_forward_sparse")
            rec(1)
            if args.fwd_only:
                return
            call(_lib.fa_backward_sparse(P[0], P[1], P[2], P[3], P[5], P[4], maskd.data_ptr(),
                                         P[6], P[7], P[8], P[9], wsb, B, H, N, d, w.scale,
                                         int(w.causal), dt, sp), "fa_backward_sparse")
            rec(2)
            return
        if args.fp8:
            call(_lib.fa_forward_fp8(*P8, P[3], P[4], B, H, N, d, w.scale, int(w.causal), sp),
                 "fa_forward_fp8")
            rec(1)
            return
        if drop:
            call(_lib.fa_forward_dropout(P[0], P[1], P[2], P[3], P[4], B, H, N, d, w.scale,
                                         int(w.causal), args.dropout, DROPOUT_SEED, dt, sp),
                 "fa_forward_dropout")
            rec(1)
            if args.fwd_only:
                return
            call(_lib.fa_backward_dropout(P[0], P[1], P[2], P[3], P[5], P[4], P[6], P[7], P[8],
                                          P[9], wsb, B, H, N, d, w.scale, int(w.causal),
                                          args.dropout, DROPOUT_SEED, dt, sp), "fa_backward_dropout")
            rec(2)
            return
        if args.splits > 1:
            call(_lib.fa_forward_split(P[0], P[1], P[2], P[3], P[4], P[9], wsb, B, H, N, d,
                                       w.scale, int(w.causal), args.splits, dt, sp),
                 "fa_forward_split")
        else:
            call(_lib.fa_forward(P[0], P[1], P[2], P[3], P[4], B, H, N, d, w.scale,
                                 int(w.causal), dt, sp), "fa_forward")
        rec(1)
        if args.fwd_only:
            return
        call(_lib.fa_backward_dq(P[0], P[1], P[2], P[3], P[5], P[4], P[9], wsb, P[6], B, H, N,
                                 d, w.scale, int(w.causal), dt, sp), "fa_backward_dq")
        rec(2)
        call(_lib.fa_backward_dkdv(P[0], P[1], P[2], P[5], P[9], wsb, P[7], P[8], B, H, N, d,
                                   w.scale, int(w.causal), dt, sp), "fa_backward_dkdv")
        rec(3)

    for _ in range(args.warmup):
        launches()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    nev = 2 if args.fwd_only else (3 if fused else 4)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        launches(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    names = (("fwd_split",) if args.splits > 1 else ("fwd_fp8",) if args.fp8 else
             ("fwd_sparse", "bwd_sparse")[: nev - 1] if sparse else
             ("fwd_dropout", "bwd_dropout")[: nev - 1] if drop else KERNELS[: nev - 1])
    per_kernel = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                  for i, n in enumerate(names)}
    step_ms = sorted(e[0].elapsed_time(e[-1]) for e in evs)

    fwd_fl, bwd_fl = credited_flops(w)
    if sparse:
        fwd_fl = 4 * w.d * mask_pairs(w, maskc)
        bwd_fl = fwd_fl * 5 // 2
    total_fl = fwd_fl if args.fwd_only else fwd_fl + bwd_fl
    tflops = total_fl / (ms_step * 1e-3) / 1e12
    dom = max(per_kernel, key=per_kernel.get)
    if sparse:
        # the forward's two contractions (fwd_sparse), or dQ's three plus dK/dV's four, per
        # visible pair of the mask
        per = 2 if dom == "fwd_sparse" else 7
        bound, amount = "mfma", per * 2 * w.d * mask_pairs(w, maskc)
    elif args.fp8:
        # the forward's two contractions per visible pair, at the fp8 peak
        bound, amount = "mfma", 4 * w.d * visible_pairs(w)
    elif drop:
        # as above, per visible (query, key) pair of the causal or full pattern
        per = 2 if dom == "fwd_dropout" else 7
        bound, amount = "mfma", per * 2 * w.d * visible_pairs(w)
    else:
        bound, amount, _ = algorithmic(w, dom, 2 if dtype_name == "bf16" else 4)
    dur_s = per_kernel[dom] * 1e-3
    if bound == "mfma":
        achieved, unit = amount / dur_s / 1e12, "TFLOP/s"
        peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    else:
        achieved, peak, unit = amount / dur_s / 1e9, PEAK_HBM_GBS, "GB/s"

    result = {
        "metric": METRIC if (args.workload == "gpt2_medium" and not args.fwd_only and not drop)
        else (f"attention {'fwd' if args.fwd_only else 'fwd+bwd'} TFLOP/s ({args.workload}"
              + (f", {args.splits} key ranges)" if args.splits > 1 else
                 f", block-sparse {args.mask} tiles{', balanced' if args.balanced else ''}, "
                 "FLOPs of visible pairs)" if sparse else
                 f", dropout {args.dropout})" if drop else
                 ", FP8 E4M3 with block scales)" if args.fp8 else ")")),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.fp8 else dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "scale": w.scale, "input_dtype": dtype_name,
                   "step": "forward" if args.fwd_only else "forward+backward",
                   **({"tile_mask": MASK_NAMES[args.mask], "visible_pairs": mask_pairs(w, maskc)}
                      if sparse else {}),
                   **({"schedule": {"seg": sched.field("SEG"),
                                    "split_rows": sched.field("N_LONG_ROWS"),
                                    "split_cols": sched.field("N_LONG_COLS"),
                                    "row_items": sched.field("N_ROWS"),
                                    "col_items": sched.field("N_COLS")}}
                      if sched is not None else {}),
                   **({"splits": args.splits} if args.splits > 1 else {}),
                   **({"dropout": args.dropout, "seed": DROPOUT_SEED} if drop else {}),
                   **({"fp8": "E4M3, power-of-two scale per 32 elements"} if args.fp8 else {})},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        **({"pct_fp8_peak": round(100.0 * tflops / PEAK_FP8_TFLOPS, 2)} if args.fp8 else {}),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
        "step_ms_min": round(step_ms[0], 4),
        "peak_mem_bytes": torch.cuda.max_memory_allocated(dev),
        "roofline": {
            "kernel": dom,
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": stored_traffic(dom, w.name),
        },
        "cpu_baseline": None,
    }
    default_run = (args.workload == "gpt2_medium" and not args.fwd_only and not fused
                   and args.splits == 1 and not args.fp8)
    if default_run and not args.no_big_d:
        result["big_d_fwd"] = big_d_forward()
    if not args.no_cpu_baseline and not fused and args.splits == 1 and not args.fp8:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
