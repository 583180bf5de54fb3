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
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 matrix peak
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


def cpu_baseline(x_bits, w_bits, n, m, budget_s=15.0):
    """The oracle, as it stands, on a bounded sample of token rows of the same layer: its
    selection (numpy, single-threaded element-wise work) and its plain C product (one fp32
    accumulator per output, ascending k, one thread), called once on the whole sample.
    BLAS thread pools are held at one thread around the call."""
    import oracle as O

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # noqa: BLE001
        threadpool_limits = None
    o, k = w_bits.shape

    def run(rows):
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                O.spmm_act(x_bits[:rows], w_bits, n, m)
                return time.perf_counter() - t0
        t0 = time.perf_counter()
        O.spmm_act(x_bits[:rows], w_bits, n, m)
        return time.perf_counter() - t0

    # two small calls size the sample (a fixed part, the weights' conversion, and a part per
    # row), then one call of about budget_s is timed
    t8, t24 = run(8), run(24)
    per_row = max((t24 - t8) / 16, 1e-4)
    rows = int(max(8, min(x_bits.shape[0], (budget_s - max(t8 - 8 * per_row, 0.0)) / per_row)))
    total_t = run(rows)
    flops = 2.0 * rows * o * k
    return {"value": round(flops / total_t / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows}/{x_bits.shape[0]} rows: 8:16 select + fp32 C product, {total_t:.1f} s"}


def gpu_time_us(torch, fn, graph, iters=10, warm=3, settle_ms=30.0):
    """Mean time per call.  graph=True: 20 calls captured in a HIP graph and replayed (the
    GPU time of short few-token calls without host launch overhead); else events around
    back-to-back calls, after at least `settle_ms` of back-to-back warmup calls (the clock
    settles under sustained matrix work) and over at least 10 ms of calls."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not graph:
        spent, n, per = 0.0, 1, 1.0
        while spent < settle_ms:
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            spent += ms
            per = max(ms / n, 1e-3)
            n = min(2 * n, 64)
        iters = max(iters, int(10.0 / per) + 1)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e3
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for _ in range(20):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 60 * 1e3


def gpu_time_rot_us(torch, fns):
    """Mean GPU time per call of a graph that cycles through `fns` (calls on distinct
    copies of the weights, so that no weight stays in the 256 MB Infinity Cache between
    its uses): max(20, len(fns)) calls per graph, three replays timed."""
    n = max(20, len(fns))
    for f in fns[:3]:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fns[0]()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for i in range(n):
                fns[i % len(fns)]()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (3 * n) * 1e3


ROT_BYTES = 600e6   # weight copies cycled per few-token row: well past the 256 MB cache


def n_copies(wbytes):
    return max(3, int(ROT_BYTES // max(wbytes, 1)) + 1)


def measure_ceilings(torch, S):
    """Achievable ceilings on this machine: streaming reads cycling over 1 GiB of distinct
    buffers (cold in the 256 MB Infinity Cache), in each of the probe's load forms (16-byte
    loads at a grid stride; contiguous blocks with 16 loads in flight per lane; direct-to-LDS
    loads like the weight streams) and over one buffer read again, and the bf16
    matrix-instruction rate on register operands, each after the clock has settled."""
    from semi_structured_sparse_amd import probe as P
    nb = 128 << 20
    bufs = [torch.empty((nb // 4,), dtype=torch.int32, device="cuda").fill_(b) for b in range(8)]
    sink = torch.empty((P.nm_probe_sink_bytes() // 4,), dtype=torch.int32, device="cuda")
    # GB/s of the three cold read forms (r0 grid stride, r1 blocks, r2 direct-to-LDS), of
    # one buffer read again (rw), and TFLOP/s of the matrix probe (mf)
    res = {}
    for mode in (0, 1, 2):
        cold = gpu_time_rot_us(torch, [(lambda b=b: P.nm_probe_read(b, nb, sink, mode=mode, check=False))
                                       for b in bufs])
        res[f"r{mode}"] = round(nb / cold / 1e3)
    warm = gpu_time_us(torch, lambda: P.nm_probe_read(bufs[0], nb, sink, mode=1, check=False), False)
    del bufs
    iters = 2000
    mf = gpu_time_us(torch, lambda: P.nm_probe_mfma(iters, sink, check=False), False)
    res.update({"rw": round(nb / warm / 1e3), "mf": round(P.nm_probe_mfma_flops(iters) / mf / 1e6)})
    log(f"ceilings: streaming read (cold, 1 GiB distinct) {res['r0']} / {res['r1']} / {res['r2']} GB/s "
        f"(grid stride / blocks / direct-to-LDS), {res['rw']} GB/s re-read; bf16 matrix instructions "
        f"{res['mf']} TFLOP/s")
    return res


def measure_rows(torch, S, synth, np, only=None):
    """Every workload row of the method's measurement table: time, dense-equivalent and
    executed TFLOP/s, algorithmic bytes and GB/s, and the fraction of the roofline that
    bounds the row (HBM for few tokens, bf16 matrix peak for many).  Few-token rows cycle
    through enough copies of their weights that each call reads its weights from HBM.
    only: row-key prefixes to measure (None: all), e.g. ["c3.", "c4.32"] for a profiler run."""

    def want(key):
        """A row key (or the prefix of a section of rows) that the selection asks for."""
        return only is None or any(key.startswith(p) or p.startswith(key) for p in only)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(
        np.int16 if a.dtype == np.uint16 else (np.int32 if a.dtype == np.int32 else np.uint8))).cuda()
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    buf = lambda nb, dt=torch.uint8: torch.empty((max(int(nb), 16),), dtype=dt, device="cuda")
    rows = {}

    def add(cfg, t, path, us, f_dense, f_exec, nbytes, bound=None, peak=PEAK_BF16_TFLOPS, key=None):
        """Log the row in full (stderr); keep [us, % of the bounding roof] under a short key
        for the JSON line.  The roof: 8 TB/s HBM for 128 tokens or fewer and the select rows,
        otherwise the bf16 matrix peak on executed FLOPs (the fp8 peak for keys ending f8
        of the lowered fp8 x fp8 rows, c3.*f8)."""
        gbps = nbytes / us / 1e3
        if bound == "hbm" or (bound is None and t <= 128):
            roof, frac = "h", gbps / PEAK_HBM_GBS
        else:
            roof, frac = ("m8" if peak == PEAK_FP8_TFLOPS else "m"), f_exec / us / 1e6 / peak
        rows[key or f"{cfg}.{t}"] = [round(us, 1) if us < 1000 else round(us), round(100 * frac, 1)]
        log(f"  {cfg:5s} T={t:5d} {path:34s} {us:9.1f} us  {f_dense / us / 1e6:8.1f} TF/s dense-eq  "
            f"{f_exec / us / 1e6:8.1f} TF/s exec  {gbps:7.0f} GB/s  {roof} {100 * frac:.1f}%  [{key or cfg}]")

    def spmm(a, ws_holder):
        nb = S.nm_spmm_workspace_size(a)
        ws_holder.append(buf(nb))
        a.workspace, a.workspace_bytes = ws_holder[-1].data_ptr(), nb
        return lambda: S.nm_spmm(a)

    def rot_spmm(make_args, weights, wbytes, ws_holder):
        """One call per weight copy (tuples of tensors, first the originals), sharing one
        workspace; make_args(*copy) builds the call's arguments."""
        cps = [weights] + [tuple(w.clone() for w in weights) for _ in range(n_copies(wbytes) - 1)]
        ws_holder.append(cps)
        args = [make_args(*c) for c in cps]
        nb = max(S.nm_spmm_workspace_size(a) for a in args)
        ws_holder.append(buf(nb))
        for a in args:
            a.workspace, a.workspace_bytes = ws_holder[-1].data_ptr(), nb
        return [(lambda a=a: S.nm_spmm(a)) for a in args]

    keep = []
    # cfg1: 2:4 activations, 64 x 512 x 512
    if want("c1.64"):
        d = synth.layer_2of4_small()
        x1, w1 = dev(d["x"]), dev(d["w"])
        y = f32(64, 512)
        fn = spmm(S.make_spmm_args(S.NM_ACT_DYNAMIC, 64, 512, 512, x1, w1, y, n=2, m=4), keep)
        add("cfg1", 64, "2:4 act (select + product)", gpu_time_us(torch, fn, True), 2.0 * 64 * 512 * 512,
            2.0 * 64 * 512 * 512, 64 * 512 * 2 + 512 * 512 * 2 + 64 * 512 * 4, key="c1.64")
    # cfg2: 8:16 activations, down-projection 4096 x 14336
    d = synth.mlp_down_8of16(t_max=8192)
    x2, w2 = dev(d["x"]), dev(d["w"])
    O2, K2 = 4096, 14336
    if want("c2.1g"):
        wk2 = dev(np.ascontiguousarray(d["w"].T))
        y = f32(1, O2)
        fns = rot_spmm(lambda wk: S.make_spmm_args(S.NM_ACT_DYNAMIC, 1, O2, K2, x2[:1], w2, y, n=8, m=16,
                                                   w_kmajor=wk), (wk2,), O2 * K2 * 2, keep)
        add("cfg2", 1, "8:16 act, K-major gather", gpu_time_rot_us(torch, fns), 2.0 * O2 * K2, 2.0 * O2 * K2 / 2,
            K2 // 2 * O2 * 2 + K2 * 2 + O2 * 4, key="c2.1g")
        keep.clear()
        del wk2
    # the select kernel alone at 8192 tokens: S(X) + mask, and values + u8 index + mask
    t = 8192
    sxb = torch.empty((t, K2), dtype=torch.int16, device="cuda")
    mk = torch.empty((t, K2 // 32), dtype=torch.int32, device="cuda")
    vv = torch.empty((t, K2 // 2), dtype=torch.int16, device="cuda")
    ix = torch.empty((t, K2 // 2), dtype=torch.uint8, device="cuda")
    if want("c2.sel"):
        fn = lambda: S.nm_sparsify(x2, 8, 16, sxb, mk, check=False)
        add("cfg2", t, "select alone: S(X) + mask", gpu_time_us(torch, fn, False), 0.0, 0.0,
            t * K2 * 2 + t * K2 * 2 + t * K2 // 8, bound="hbm", key="c2.sel")
    if want("c2.cmp"):
        fn = lambda: S.nm_compress(x2, 8, 16, vv, ix, S.NM_META_U8, mask=mk, check=False)
        add("cfg2", t, "select alone: values + u8 idx + mask", gpu_time_us(torch, fn, False), 0.0, 0.0,
            t * K2 * 2 + t * K2 // 2 * 3 + t * K2 // 8, bound="hbm", key="c2.cmp")
    if want("c2.selsc"):
        # scored selection: activations weighted by the fp32 L2 norm of each weight column
        cs = w2.view(torch.bfloat16).float().pow(2).sum(0).sqrt().contiguous()
        fn = lambda: S.nm_sparsify_scored(x2, 8, 16, cs, S.NM_SCORE_ACT_WEIGHTED, sxb, mk, check=False)
        add("cfg2", t, "select alone, |x| * weight-column norm: S(X) + mask", gpu_time_us(torch, fn, False), 0.0,
            0.0, t * K2 * 2 + t * K2 * 2 + t * K2 // 8 + K2 * 4, bound="hbm", key="c2.selsc")
        del cs
    if want("c2.selpts"):
        # the mitigated selection (D-PTS + VAR): row mean, shift, select, variance factor
        mu_, al_ = f32(t), f32(t)
        fn = lambda: S.nm_sparsify_pts(x2, 8, 16, S.NM_PTS_DYNAMIC | S.NM_PTS_VAR, sxb, mk, None, mu_, al_,
                                       check=False)
        add("cfg2", t, "select alone, D-PTS + VAR: S(x~) + mask", gpu_time_us(torch, fn, False), 0.0, 0.0,
            t * K2 * 2 + t * K2 * 2 + t * K2 // 8 + 2 * t * 4, bound="hbm", key="c2.selpts")
    del sxb, mk, vv, ix
    for t in (1, 16, 128, 2048, 8192):
        if not want(f"c2.{t}"):
            continue
        y = f32(t, O2)
        f = 2.0 * t * O2 * K2
        if t <= 128:
            fns = rot_spmm(lambda w: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, O2, K2, x2[:t], w, y, n=8, m=16),
                           (w2,), O2 * K2 * 2, keep)
            us = gpu_time_rot_us(torch, fns)
        else:
            us = gpu_time_us(torch, spmm(S.make_spmm_args(S.NM_ACT_DYNAMIC, t, O2, K2, x2[:t], w2, y, n=8, m=16),
                                         keep), False)
        add("cfg2", t, "8:16 act (select + product)", us, f, f, t * K2 * 2 + O2 * K2 * 2 + t * O2 * 4, key=f"c2.{t}")
        keep.clear()
    # the same layer with the mitigations (D-PTS + VAR) inside the call
    v2 = f32(O2)
    S.nm_weight_sums(w2, v2)
    for t in (1, 128, 8192):
        if not want(f"c2.{t}pts"):
            continue
        y = f32(t, O2)
        f = 2.0 * t * O2 * K2
        mkp = lambda w: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, O2, K2, x2[:t], w, y, n=8, m=16,
                                         pts=S.NM_PTS_DYNAMIC | S.NM_PTS_VAR, col_shift=v2)
        if t <= 128:
            us = gpu_time_rot_us(torch, rot_spmm(mkp, (w2,), O2 * K2 * 2, keep))
        else:
            us = gpu_time_us(torch, spmm(mkp(w2), keep), False)
        add("cfg2", t, "8:16 act, D-PTS + VAR (select + product)", us, f, f,
            t * K2 * 2 + O2 * K2 * 2 + t * O2 * 4 + O2 * 4, key=f"c2.{t}pts")
        keep.clear()
    del x2, w2
    # cfg3: 6:8 weights lowered to 2:4, 4096 x 4096, lifted activations
    d = synth.slide_6of8_layer(t_max=4096)
    w3, x3 = dev(d["w"]), dev(d["x"])
    v = torch.empty((4096, 3072), dtype=torch.int16, device="cuda")
    i8 = torch.empty((4096, 3072), dtype=torch.uint8, device="cuda")
    S.nm_compress(w3, 6, 8, v, i8, S.NM_META_U8)
    vp = torch.empty((4096, 3072), dtype=torch.int16, device="cuda")
    mp = torch.empty((4096, 768), dtype=torch.uint8, device="cuda")
    S.nm_lower_slide(v, i8, 4096, 4096, 4, vp, mp, S.NM_META_2BIT)
    for t in (1, 16, 128, 4096):
        if not want(f"c3.{t}"):
            continue
        y = f32(t, 4096)
        mk3 = lambda v_, m_: S.make_spmm_args(S.NM_W_SLIDE, t, 4096, 4096, x3[:t], v_, y, ns=4, w_meta=m_,
                                              w_meta_fmt=S.NM_META_2BIT)
        if t <= 128:
            us = gpu_time_rot_us(torch, rot_spmm(mk3, (vp, mp), 4096 * 3072 * 2 + 4096 * 768, keep))
        else:
            us = gpu_time_us(torch, spmm(mk3(vp, mp), keep), False)
        add("cfg3", t, "6:8 W lowered to 2:4, lifted X", us, 2.0 * t * 4096 * 4096,
            2.0 * t * 4096 * 3072, 4096 * 3072 * 2 + 4096 * 768 + t * 4096 * 2 + t * 4096 * 4, key=f"c3.{t}")
        keep.clear()
    # the same layer with fp8 weights (per-row codes, the input format) and activations
    # quantized per token to fp8 inside the call (fused with the lift), on the fp8 sparse
    # matrix instruction; prefill measured against the fp8 dense peak
    q8, s8 = synth.fp8_e4m3_quantize_rows(vp.cpu().numpy().view(np.uint16))
    q8d, s8d = dev(q8), torch.from_numpy(s8).cuda()
    wb8 = 4096 * 3072 + 4096 * 768 + 4096 * 4
    for t in (1, 16, 128, 4096):
        if not want(f"c3.{t}f8"):
            continue
        y = f32(t, 4096)
        mk8 = lambda q_, s_, m_: S.make_spmm_args(S.NM_W_SLIDE, t, 4096, 4096, x3[:t], q_, y, ns=4,
                                                  w_dtype=S.NM_W_FP8E4M3, w_scale=s_, w_meta=m_,
                                                  w_meta_fmt=S.NM_META_2BIT)
        if t <= 128:
            us = gpu_time_rot_us(torch, rot_spmm(mk8, (q8d, s8d, mp), wb8, keep))
        else:
            us = gpu_time_us(torch, spmm(mk8(q8d, s8d, mp), keep), False)
        add("cfg3", t, "6:8 lowered, fp8 W + per-token fp8 X", us, 2.0 * t * 4096 * 4096, 2.0 * t * 4096 * 3072,
            wb8 + t * 4096 * 2 + t * 4096 * 4, peak=PEAK_FP8_TFLOPS, key=f"c3.{t}f8")
        keep.clear()
    del q8d, s8d
    del w3, x3, v, i8, vp, mp
    # cfg4: hybrid, 14336 x 4096, 25% dense columns
    d = synth.hybrid_up_layer(t_max=2048)
    w4, x4 = dev(d["w"]), dev(d["x"])
    o4, k4 = d["w"].shape
    kd = d["k_dense"]
    ks = k4 - kd
    sc = torch.empty((ks,), dtype=torch.int32, device="cuda")
    dc = torch.empty((kd,), dtype=torch.int32, device="cuda")
    wv = torch.empty((o4, ks // 2), dtype=torch.int16, device="cuda")
    wm = torch.empty((o4, ks // 8), dtype=torch.uint8, device="cuda")
    wd = torch.empty((o4, kd), dtype=torch.int16, device="cuda")
    S.nm_hybrid_pack(w4, kd, sc, dc, wv, wm, S.NM_META_2BIT, wd, buf(S.nm_hybrid_pack_workspace_size(k4)))
    wb4 = o4 * ks + o4 * ks // 8 + o4 * kd * 2
    for t in (1, 8, 32, 64, 2048):
        if not want(f"c4.{t}"):
            continue
        y = f32(t, o4)
        nb = S.nm_hybrid_gemm_workspace_size(t, ks, kd, o4, True)
        wsb = buf(nb)
        xs = x4[:t]
        call = lambda wv_, wm_, wd_: (lambda: S.nm_hybrid_gemm(xs, sc, ks, dc, kd, wv_, wm_, S.NM_META_2BIT, wd_, o4,
                                                               y, workspace=wsb, workspace_bytes=nb))
        if t <= 128:
            cps = [(wv, wm, wd)] + [(wv.clone(), wm.clone(), wd.clone()) for _ in range(n_copies(wb4) - 1)]
            us = gpu_time_rot_us(torch, [call(*c) for c in cps])
            del cps
        else:
            us = gpu_time_us(torch, call(wv, wm, wd), False)
        add("cfg4", t, "hybrid 2:4 + 25% dense columns", us, 2.0 * t * o4 * k4,
            2.0 * t * o4 * (kd + ks / 2), wb4 + t * k4 * 2 + t * o4 * 4, key=f"c4.{t}")
    del w4, x4, sc, dc, wv, wm, wd
    if not (want("c5.") or want("sp.")):
        return rows
    # cfg5: one 8B-shaped layer, 16:32 and 8:16, bf16 and fp8 weights, T = 64 and 8192
    lay = synth.transformer_layer(t_max=8192, with_fp8=True)
    names = list(synth.TRANSFORMER_SHAPES)
    wdev = {nm: dev(lay["w"][nm]) for nm in names}
    w8dev = {nm: (dev(lay["w8"][nm]), torch.from_numpy(lay["s8"][nm]).cuda()) for nm in names}
    xdev = {st: dev(v) for st, v in lay["x"].items()}
    del lay
    for t in (64, 8192):
        for n, m in ((16, 32), (8, 16)):
            for kind in ("bf16", "fp8"):
                if not want(f"c5.{t}.{m}{'f8' if kind == 'fp8' else ''}s"):
                    continue
                tot_us = tot_f = tot_b = 0.0
                for nm in names:
                    o_, k_, st = synth.TRANSFORMER_SHAPES[nm]
                    y = f32(t, o_)
                    xin = xdev[st][:t]
                    if kind == "bf16":
                        mk5 = lambda w_: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o_, k_, xin, w_, y, n=n, m=m)
                        wts = (wdev[nm],)
                        wb = o_ * k_ * 2
                    else:
                        mk5 = lambda q_, s_: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o_, k_, xin, q_, y, n=n, m=m,
                                                              w_dtype=S.NM_W_FP8E4M3, w_scale=s_)
                        wts = w8dev[nm]
                        wb = o_ * k_ + o_ * 4
                    if t <= 128:
                        tot_us += gpu_time_rot_us(torch, rot_spmm(mk5, wts, wb, keep))
                    else:
                        tot_us += gpu_time_us(torch, spmm(mk5(*wts), keep), False, iters=5, warm=2)
                    tot_f += 2.0 * t * o_ * k_
                    tot_b += wb + t * k_ * 2 + t * o_ * 4
                    keep.clear()
                add("cfg5", t, f"layer {n}:{m} act, {kind} W", tot_us, tot_f, tot_f, tot_b,
                    key=f"c5.{t}.{m}{'f8' if kind == 'fp8' else ''}s")
    # the same layer with the linears that share an input concatenated along the output
    # dimension (q|k|v: 6144 x 4096, gate|up: 28672 x 4096): four calls instead of seven,
    # one selection per input stream, identical outputs
    groups = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))
    wcat = {g: torch.cat([wdev[nm] for nm in parts], 0).contiguous() for g, parts in groups}
    w8cat = {g: (torch.cat([w8dev[nm][0] for nm in parts], 0).contiguous(),
                 torch.cat([w8dev[nm][1] for nm in parts], 0).contiguous()) for g, parts in groups}
    del wdev, w8dev
    for t in (64, 8192):
        for n, m in ((16, 32), (8, 16)):
            for kind in ("bf16", "fp8"):
                if not want(f"c5.{t}.{m}{'f8' if kind == 'fp8' else ''}c"):
                    continue
                tot_us = tot_f = tot_b = 0.0
                for g, parts in groups:
                    o_ = sum(synth.TRANSFORMER_SHAPES[nm][0] for nm in parts)
                    _, k_, st = synth.TRANSFORMER_SHAPES[parts[0]]
                    y = f32(t, o_)
                    xin = xdev[st][:t]
                    if kind == "bf16":
                        mk5 = lambda w_: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o_, k_, xin, w_, y, n=n, m=m)
                        wts = (wcat[g],)
                        wb = o_ * k_ * 2
                    else:
                        mk5 = lambda q_, s_: S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o_, k_, xin, q_, y, n=n, m=m,
                                                              w_dtype=S.NM_W_FP8E4M3, w_scale=s_)
                        wts = w8cat[g]
                        wb = o_ * k_ + o_ * 4
                    if t <= 128:
                        tot_us += gpu_time_rot_us(torch, rot_spmm(mk5, wts, wb, keep))
                    else:
                        tot_us += gpu_time_us(torch, spmm(mk5(*wts), keep), False, iters=5, warm=2)
                    tot_f += 2.0 * t * o_ * k_
                    tot_b += wb + t * k_ * 2 + t * o_ * 4
                    keep.clear()
                add("cfg5", t, f"layer {n}:{m} act, {kind} W, fused qkv + gate|up", tot_us, tot_f, tot_f, tot_b,
                    key=f"c5.{t}.{m}{'f8' if kind == 'fp8' else ''}c")
    # Spense MLP of the same layer: 25% of the intermediate indices dense, chosen by the
    # loss-aware score (Hessian roots from the layer's input streams) and moved to the end;
    # gate|up as one output-split call (rows [gate_s, up_s, gate_d, up_d]), down as an
    # input-split call on its input in the permuted order.  Packing is offline (untimed);
    # the GLU's elementwise product between the two calls is not part of the timed path.
    i_n, hd = 14336, 4096
    wgu, wdn = wcat["gate_up"], wcat["down"]
    hs_in = xdev["mlp_in"].view(torch.bfloat16).double().pow(2).sum(0).sqrt().contiguous()
    hs_mid = xdev["down_in"].view(torch.bfloat16).double().pow(2).sum(0).sqrt().contiguous()
    n_dense = i_n // 4
    ns = i_n - n_dense
    perm = torch.empty((i_n,), dtype=torch.int32, device="cuda")
    S.nm_spense_glu_order(wgu[:i_n], wgu[i_n:], wdn, hs_in, hs_mid, n_dense, S.NM_SPENSE_LOSS, perm,
                          buf(S.nm_spense_glu_order_workspace_size(i_n)))
    perm_gu = torch.cat([perm[:ns], perm[:ns] + i_n, perm[ns:], perm[ns:] + i_n]).to(torch.int32).contiguous()
    o_s, o_d = 2 * ns, 2 * n_dense
    gv = torch.empty((o_s, hd // 2), dtype=torch.int16, device="cuda")
    gm = torch.empty((o_s, hd // 8), dtype=torch.uint8, device="cuda")
    gd = torch.empty((o_d, hd), dtype=torch.int16, device="cuda")
    S.nm_spense_pack(wgu, 0, perm_gu, o_s, gv, gm, S.NM_META_2BIT, gd,
                     buf(S.nm_spense_pack_workspace_size(2 * i_n, hd, 0, o_s)))
    dv = torch.empty((hd, ns // 2), dtype=torch.int16, device="cuda")
    dm = torch.empty((hd, ns // 8), dtype=torch.uint8, device="cuda")
    dd = torch.empty((hd, n_dense), dtype=torch.int16, device="cuda")
    S.nm_spense_pack(wdn, 1, perm, ns, dv, dm, S.NM_META_2BIT, dd)
    torch.cuda.synchronize()
    del wcat, w8cat
    wbytes = o_s * hd + o_s * hd // 8 + o_d * hd * 2 + hd * ns + hd * ns // 8 + hd * n_dense * 2
    packed = (gv, gm, gd, dv, dm, dd)
    for t in (1, 64, 2048):
        if not want(f"sp.{t}"):
            continue
        xg, a_in = xdev["mlp_in"][:t], xdev["down_in"][:t]   # down's input: the permuted GLU output's shape
        ygu, yd = f32(t, 2 * i_n), f32(t, hd)
        cps = [packed] + ([tuple(z.clone() for z in packed) for _ in range(n_copies(wbytes) - 1)] if t <= 128 else [])
        keep.append(cps)
        nb1 = S.nm_spense_outsplit_workspace_size(t, hd, o_s, o_d)
        nb2 = S.nm_hybrid_gemm_workspace_size(t, ns, n_dense, hd, False)
        ws = buf(max(nb1, nb2))
        keep.append(ws)

        def mlp(c, xg=xg, a_in=a_in, ygu=ygu, yd=yd, ws=ws, nb1=nb1, nb2=nb2):
            S.nm_spense_outsplit_gemm(xg, c[0], c[1], o_s, c[2], o_d, ygu, 0, ws, workspace_bytes=nb1, check=False)
            S.nm_hybrid_gemm(a_in, None, ns, None, n_dense, c[3], c[4], S.NM_META_2BIT, c[5], hd, yd, 0,
                             workspace=ws, workspace_bytes=nb2, check=False)
        fns = [(lambda c=c: mlp(c)) for c in cps]
        us = gpu_time_rot_us(torch, fns) if t <= 128 else gpu_time_us(torch, fns[0], False)
        f_dense = 2.0 * t * (2 * i_n * hd + hd * i_n)
        f_exec = 2.0 * t * (o_s * hd / 2 + o_d * hd + hd * ns / 2 + hd * n_dense)
        nbytes = wbytes + t * hd * 2 + t * 2 * i_n * 4 + t * i_n * 2 + t * hd * 4
        add("spense", t, "MLP: gate|up output-split + down input-split, 25% dense", us, f_dense, f_exec, nbytes,
            key=f"sp.{t}")
        keep.clear()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults reach the sustained clock: under back-to-back matrix work the chip's power
    # control lowers the clock for the first ~25 steps (product kernel 720 -> 980 -> 700 us)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-workload rows (all five workloads at their token counts)")
    ap.add_argument("--rows-only", default=None,
                    help="comma-separated row-key prefixes: measure only those rows and print them (no headline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB five times (counter calibration)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor bf16 GEMM (torch.mm) on the headline shape, fp32 and bf16 output")
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
    if args.vendor_gemm:
        # context for the product kernel: the library GEMM on the same operands (dense bf16,
        # no selection), timed like the headline product after the clock has settled
        d = synth.mlp_down_8of16(t_max=args.tokens)
        xb = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
        wt = torch.from_numpy(d["w"].view(np.int16)).cuda().view(torch.bfloat16).t()
        f = 2.0 * xb.shape[0] * wt.shape[1] * xb.shape[1]
        res = {}
        for name, fn in (("fp32_out", lambda: torch.mm(xb, wt, out_dtype=torch.float32)),
                         ("bf16_out", lambda: torch.mm(xb, wt))):
            us = gpu_time_us(torch, fn, False, settle_ms=60.0)
            res[name] = {"us": round(us, 1), "TFLOP/s": round(f / us / 1e6, 1)}
            log(f"vendor GEMM {name}: {us:.1f} us, {f / us / 1e6:.1f} TFLOP/s")
        print(json.dumps({"vendor_gemm": res, "tokens": int(xb.shape[0])}), flush=True)
        return
    S.lib()
    if args.rows_only is not None:
        rows = measure_rows(torch, S, synth, np, only=[p for p in args.rows_only.split(",") if p])
        print(json.dumps({"rows": rows}, separators=(",", ":")), flush=True)
        return
    extra = {}
    if not args.no_rows:
        # the per-workload rows and the machine ceilings run first: the headline steps are
        # then timed on a GPU whose clock has settled under sustained work
        extra["ceil"] = measure_ceilings(torch, S)
        log("per-workload rows:")
        extra["rows"] = measure_rows(torch, S, synth, np)
        torch.cuda.synchronize()
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
        "config": {"workload": f"8:16 act-sparse down-proj X {T}x{K} t(4)*.5, W {O_}x{K} N(0,.02)", "tokens": T,
                   "pattern": "8:16"},
        "kernels": {"select_us": round(sel_ms * 1e3, 1), "product_us": round(gemm_ms * 1e3, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    result.update(extra)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_bits, w_bits, n, m)
    print(json.dumps(result, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
