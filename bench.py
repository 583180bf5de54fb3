#!/usr/bin/env python3
"""Benchmark of the N:M activation-sparse linear layer on one MI355X.

Workload (the down-projection layer the throughput metric is quoted on): 8:16 activation
sparsity, X 8192 x 14336 bf16 drawn Student-t(4) * 0.5, W 4096 x 14336 bf16 ~ N(0, 0.02),
Y = S(X) . W^T in fp32.  One step = the whole hot path over one batch:
  nm_sparsify  (per-group top-8 of 16 by magnitude -> S(X), pruned entries +0)
  nm_spmm      (ACT_MASKED with S(X): the selected X contracted with W on matrix cores)
Inputs are resident in HBM before the timed region.  Prints ONE JSON line on stdout.

--gpus N with N > 1 is refused: this build runs on a single GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PMC_FILE = os.path.join(ROOT, "profiles", "gemm_lds_pmc.json")
PMC_SOURCES = ["semi_structured_sparse_amd/csrc/gemm_lds.hip", "semi_structured_sparse_amd/csrc/nm_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(tokens):
    """HBM bytes per launch of the product kernel from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration); None if absent or
    taken on a different kernel source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha") != source_sha(PMC_SOURCES) or d.get("tokens") != tokens:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(x_bits, w_bits, n, m, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of token rows of the same layer."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
    rows = 32
    t0 = time.perf_counter()
    O.spmm_act(x_bits[:rows], w_bits, n, m)
    dt = time.perf_counter() - t0
    total_rows, total_t = rows, dt
    # grow the sample until about budget_s of CPU work has been timed
    while total_t < budget_s and total_rows < x_bits.shape[0]:
        r = int(min(max(rows * 2, 32), x_bits.shape[0] - total_rows, 4096))
        if r <= 0:
            break
        t0 = time.perf_counter()
        O.spmm_act(x_bits[total_rows:total_rows + r], w_bits, n, m)
        total_t += time.perf_counter() - t0
        total_rows += r
        rows = r
    o, k = w_bits.shape
    flops = 2.0 * total_rows * o * k
    return {"value": round(flops / total_t / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{total_rows} of {x_bits.shape[0]} token rows of the same 8:16 layer "
                      f"(numpy fp64 select + matmul), {total_t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shapes", action="store_true", help="also time the decode token counts (stderr + JSON)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on exactly one GPU; --gpus N > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import semi_structured_sparse_amd as S
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return
    S.lib()
    n, m = 8, 16
    d = synth.mlp_down_8of16(t_max=args.tokens)
    x_bits, w_bits = d["x"], d["w"]
    T, K = x_bits.shape
    O_ = w_bits.shape[0]
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    w = torch.from_numpy(w_bits.view(np.int16)).cuda()
    y = torch.empty((T, O_), dtype=torch.float32, device="cuda")
    sx = torch.empty((T, K), dtype=torch.int16, device="cuda")
    a = S.make_spmm_args(S.NM_ACT_MASKED, T, O_, K, sx, w, y, n=n, m=m)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        S.nm_sparsify(x, n, m, sx, None)
        if ev is not None:
            ev[1].record()
        S.nm_spmm(a)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    gemm_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * T * O_ * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    sel_bytes = T * K * 2 * 2
    log(f"step {ms_per_step:.3f} ms: select {sel_ms * 1e3:.1f} us ({sel_bytes / sel_ms / 1e6:.0f} GB/s), "
        f"product {gemm_ms * 1e3:.1f} us ({achieved:.1f} TFLOP/s)")
    traffic = measured_traffic(T)

    result = {
        "metric": "N:M sparsify+SpMM TFLOP/s (dense-equiv & executed), GB/s, % MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"8:16 activation-sparse MLP down-projection, X {T}x{K} Student-t(4)*0.5, "
                               f"W {O_}x{K} N(0,0.02), fp32 out", "tokens": T, "in_features": K,
                   "out_features": O_, "pattern": "8:16", "route": "nm_sparsify -> S(X), nm_spmm(ACT_MASKED)"},
        "executed_tflops": round(value, 2),
        "kernels": {
            "select_us": round(sel_ms * 1e3, 2), "select_GBps": round(sel_bytes / sel_ms / 1e6, 1),
            "select_frac_hbm": round(sel_bytes / sel_ms / 1e6 / PEAK_HBM_GBS, 4),
            "product_us": round(gemm_ms * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }

    if args.shapes:
        shapes = {}
        for tt in (1, 16, 128, 2048):
            ys = torch.empty((tt, O_), dtype=torch.float32, device="cuda")
            ad = S.make_spmm_args(S.NM_ACT_DYNAMIC, tt, O_, K, x[:tt], w, ys, n=n, m=m)
            nb = S.nm_spmm_workspace_size(ad)
            wsb = torch.empty((max(nb, 16),), dtype=torch.uint8, device="cuda")
            ad.workspace, ad.workspace_bytes = wsb.data_ptr(), nb
            for _ in range(3):
                S.nm_spmm(ad)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            it = 20
            e0.record()
            for _ in range(it):
                S.nm_spmm(ad)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / it * 1e3
            byts = tt * K * 2 + O_ * K * 2 + tt * O_ * 4
            shapes[str(tt)] = {"us": round(us, 2), "TFLOPs": round(2.0 * tt * O_ * K / us / 1e6, 2),
                               "GBps": round(byts / us / 1e3, 1)}
            log(f"T={tt}: {us:.1f} us, {2.0 * tt * O_ * K / us / 1e6:.2f} TFLOP/s, {byts / us / 1e3:.0f} GB/s")
        result["shapes"] = shapes

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_bits, w_bits, n, m)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
