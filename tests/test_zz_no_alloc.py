"""The no-allocation entry point (nm_spmm_noalloc) against nm_spmm with a caller
workspace: the same kernels, so the same bits, on routes that use scratch (staged S(X),
split partial sums, lifted X, K-blocked positions, fp8 quantized tokens, the mitigated
selection), two calls in a row with the second smaller; a call too large for the buffer
is refused before any work is enqueued."""
import numpy as np
import pytest

import oracle as O
import synth
from nm_testutil import check_gemm, dev, empty, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import semi_structured_sparse_amd as S  # noqa: E402


def sync():
    torch.cuda.synchronize()


def both(make):
    """make(y) -> args (no workspace).  Returns (y_noalloc, y_workspace, taken_noalloc)."""
    ya = make(None)
    y1 = ya[0]
    a = ya[1]
    S.nm_spmm_noalloc(a)
    sync()
    t_no = S.route_taken(a)
    y2, b = make(None)
    nb = S.nm_spmm_workspace_size(b)
    ws = empty((max(nb, 16),), np.uint8)
    b.workspace, b.workspace_bytes = ws.data_ptr(), nb
    S.nm_spmm(b)
    sync()
    return host(y1, np.float32), host(y2, np.float32), S.taken_names(t_no), S.taken_names(S.route_taken(b))


def act_case(t, o, k, n, m, x, w, w8=None, s8=None, pts=0, v=None):
    def make(_):
        y = empty((t, o), np.float32, fill=float("nan"))
        if w8 is None:
            a = S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o, k, dev(x), dev(w), y, n=n, m=m, pts=pts, col_shift=v)
        else:
            a = S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o, k, dev(x), dev(w8), y, n=n, m=m, w_dtype=S.NM_W_FP8E4M3,
                                 w_scale=dev(s8), pts=pts, col_shift=v)
        return y, a
    return make


def test_noalloc_matches_workspace_calls():
    print("noalloc act", flush=True)
    rng = np.random.default_rng(90)
    k, o = 4096, 2048
    x = synth.student_t_bf16(rng, (600, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    for t in (600, 64, 16, 1):          # larger first, then smaller: the buffer keeps old contents
        y1, y2, tk1, tk2 = both(act_case(t, o, k, 8, 16, x[:t], w))
        assert tk1 == tk2, (t, tk1, tk2)
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), f"act t={t}"
        sx, _ = O.sparsify(x[:t], 8, 16)
        check_gemm(y1, O.gemm(sx, w), sx, w, label=f"noalloc act t={t}")
    assert "select" in tk1 or "few_select" in tk1


def test_noalloc_sparse_weights_and_fp8():
    print("noalloc sparse / fp8", flush=True)
    rng = np.random.default_rng(91)
    k, o = 4096, 2048
    x = synth.normal_bf16(rng, (300, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    v, i = O.compress(w, 6, 8)
    vp, ip = O.slide_lower(v, i, k, 4)
    mp = O.pack_meta_2bit(ip)
    pr, _ = O.sparsify(w, 6, 8)
    for t in (300, 128, 40):
        def make(_, t=t):
            y = empty((t, o), np.float32, fill=float("nan"))
            return y, S.make_spmm_args(S.NM_W_SLIDE, t, o, k, dev(x[:t]), dev(vp), y, ns=4, w_meta=dev(mp),
                                       w_meta_fmt=S.NM_META_2BIT)
        y1, y2, tk1, tk2 = both(make)
        assert tk1 == tk2
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), f"slide t={t}"
        check_gemm(y1, O.gemm(x[:t], pr), x[:t], pr, label=f"noalloc slide t={t}")
    q, sc = synth.fp8_e4m3_quantize_rows(w)
    for t in (128, 64):
        y1, y2, tk1, tk2 = both(act_case(t, o, k, 16, 32, x[:t], None, q, sc))
        assert tk1 == tk2
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), f"fp8 t={t}"


def test_noalloc_mitigated_selection():
    print("noalloc pts", flush=True)
    rng = np.random.default_rng(92)
    k, o = 2048, 1024
    x = synth.student_t_bf16(rng, (200, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    vv = empty((o,), np.float32)
    S.nm_weight_sums(dev(w), vv)
    pts = S.NM_PTS_DYNAMIC | S.NM_PTS_VAR
    for t in (200, 33):
        y1, y2, tk1, tk2 = both(act_case(t, o, k, 8, 16, x[:t], w, pts=pts, v=vv))
        assert tk1 == tk2
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), f"pts t={t}"


def test_noalloc_without_the_large_split():
    """A call whose preferred route splits the reduction of its 256 x 256 tiles with more
    scratch than the buffer holds (2:4 weights, 4096 x 14336, 2048 tokens: K-blocked
    positions, then partial tiles) runs those tiles unsplit: every output written, one row
    of every 256-row band and the last within tolerance of the oracle, as nm_spmm's split
    route is."""
    t, o, k = 2048, 4096, 14336
    rng = np.random.default_rng(93)
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    v = torch.empty((o, k // 2), dtype=torch.int16, device="cuda")
    mt = torch.empty((o, k // 8), dtype=torch.uint8, device="cuda")
    S.nm_compress(dev(w), 2, 4, v, mt, S.NM_META_2BIT)
    sync()
    xd = dev(x)

    def make(_):
        y = empty((t, o), np.float32, fill=float("nan"))
        return y, S.make_spmm_args(S.NM_W_COMPRESSED, t, o, k, xd, v, y, w_meta=mt, w_meta_fmt=S.NM_META_2BIT)

    assert S.nm_spmm_workspace_size(make(None)[1]) > S.NM_NOALLOC_SCRATCH_BYTES
    y1, y2, tk1, tk2 = both(make)
    assert "tile_split" in tk2 and "tile_split" not in tk1, (tk1, tk2)
    rows = np.unique(np.r_[np.arange(0, t, 256) + rng.integers(0, 256, t // 256), t - 1])
    pr, _ = O.sparsify(w, 2, 4)
    ref = O.gemm(x[rows], pr)
    for yy, lab in ((y1, "noalloc unsplit"), (y2, "workspace split")):
        assert np.isfinite(yy).all(), lab
        check_gemm(yy[rows], ref, x[rows], pr, label=lab)


def test_noalloc_refuses_oversized_calls():
    t, o, k = 8192, 4096, 14336
    xd = torch.zeros((t, k), dtype=torch.int16, device="cuda")
    wd = torch.zeros((o, k), dtype=torch.int16, device="cuda")
    y = torch.full((t, o), 7.0, dtype=torch.float32, device="cuda")
    a = S.make_spmm_args(S.NM_ACT_DYNAMIC, t, o, k, xd, wd, y, n=8, m=16)
    assert S.nm_spmm_workspace_size(a) > S.NM_NOALLOC_SCRATCH_BYTES
    assert S.nm_spmm_noalloc(a, check=False) == S.NM_ESCRATCH
    sync()
    assert bool((y == 7.0).all().item()), "a refused call wrote its output"
