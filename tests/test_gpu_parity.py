"""GPU <-> oracle parity through the C ABI (needs an MI355X and the built library).

Integer / byte work (masks, S(X), compressed values, index bytes, 2-bit metadata,
lowered windows, hybrid column lists and packed weights) must match the oracle bit for
bit.  Products must meet: relative Frobenius error <= 1e-3 and per element
|err| <= 1e-2 * (|A|.|B|) + 1e-4 against the oracle's fp32-accumulated result on the same
bf16 inputs.  Full-size products are checked on one row of every band of output rows
against the oracle, for unwritten outputs everywhere, and through random projections of
the whole output (nm_testutil).

Kernel routes are chosen through the calls' route hints: a `with use_route(...)` block
sets the hints that the helpers below put into every call they make.
"""
import numpy as np
import pytest

import oracle as O
import synth
from nm_testutil import (band_rows, check_all_written, check_gemm, check_gemm_vals, check_projection, dev, empty,
                         host, sample_rows)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import semi_structured_sparse_amd as S  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    S.lib()
    yield
    torch.cuda.synchronize()


def sync():
    torch.cuda.synchronize()


# Route hints (and tuning values) for the calls made inside a `with use_route(...)` block,
# and the route report of the last call made by the helpers below.  This is test-side
# state: the library reads nothing but its arguments.
_ROUTE = {"route": 0, "few_wpb": 0, "few_splits": 0, "tile_wg": 0}
LAST_TAKEN = [0]


class use_route:
    """Hints named as in S.ROUTE; blocks nest (bits are OR-ed, tuning values override)."""

    def __init__(self, *names, few_wpb=0, few_splits=0, tile_wg=0):
        self.bits = S.route_bits(*names)
        self.tune = {"few_wpb": few_wpb, "few_splits": few_splits, "tile_wg": tile_wg}

    def __enter__(self):
        self.old = dict(_ROUTE)
        _ROUTE["route"] |= self.bits
        for k, v in self.tune.items():
            if v:
                _ROUTE[k] = v
        return self

    def __exit__(self, *exc):
        _ROUTE.clear()
        _ROUTE.update(self.old)


def mk_args(*a, **kw):
    """S.make_spmm_args with the current route hints (an explicit route= is OR-ed in)."""
    kw["route"] = kw.get("route", 0) | _ROUTE["route"]
    for k in ("few_wpb", "few_splits", "tile_wg"):
        kw.setdefault(k, _ROUTE[k])
    return S.make_spmm_args(*a, **kw)


def spmm_call(a):
    S.nm_spmm(a)
    LAST_TAKEN[0] = S.route_taken(a)


def taken():
    """NM_TAKEN_* names reported by the last helper call."""
    return S.taken_names(LAST_TAKEN[0])


def special_rows(k, rng):
    """Rows full of ties, signed zeros, subnormals, infinities and NaN."""
    rows = [np.full(k, 0x3F80, np.uint16),                       # all equal
            np.where(rng.random(k) < 0.5, 0x8000, 0x0000).astype(np.uint16),
            rng.choice(np.array([0x0001, 0x0002, 0x8001, 0x0080, 0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80, 0],
                                np.uint16), size=k),
            rng.choice(np.array([0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x4000], np.uint16), size=k)]
    return np.stack(rows)


# --------------------------------------------------------------------- select ---

SELECT_CASES = [(2, 4), (1, 4), (3, 4), (4, 8), (6, 8), (1, 8), (8, 16), (5, 16), (16, 32), (1, 32), (31, 32),
                (4, 4), (32, 32)]


@pytest.mark.parametrize("n,m", SELECT_CASES)
@pytest.mark.parametrize("rows,groups,pad", [(37, 131, 0), (5, 3, 8), (1, 64, 16), (70, 64, 0)])
def test_select_bitexact(n, m, rows, groups, pad):
    print(f"select n={n} m={m} rows={rows} groups={groups} pad={pad}", flush=True)
    rng = np.random.default_rng(1000 * m + n + rows)
    k = groups * m
    x = synth.student_t_bf16(rng, (rows, k), 4.0, 0.5)
    x[: min(4, rows)] = special_rows(k, rng)[: min(4, rows)]
    ld = k + pad
    xd = dev(x, ld)
    y = empty((rows, ld), np.uint16, fill=-1)
    words = (k + 31) // 32
    mask = empty((rows, words), np.uint32, fill=-1)
    S.nm_sparsify(xd, n, m, y, mask, k=k)
    kc = k * n // m
    vals = empty((rows, kc), np.uint16, fill=-1)
    idx = empty((rows, kc), np.uint8, fill=255)
    mask2 = empty((rows, words), np.uint32, fill=-1)
    S.nm_compress(xd, n, m, vals, idx, S.NM_META_U8, mask2, k=k)
    sync()
    s_ref, keep = O.sparsify(x, n, m)
    v_ref, i_ref = O.compress(x, n, m)
    m_ref = O.pack_mask(keep)
    assert (host(y, np.uint16)[:, :k] == s_ref).all()
    assert (host(y, np.uint16)[:, k:] == 0xFFFF).all()          # padding untouched
    assert (host(mask, np.uint32) == m_ref).all()
    assert (host(mask2, np.uint32) == m_ref).all()
    assert (host(vals, np.uint16) == v_ref).all()
    assert (host(idx, np.uint8) == i_ref).all()
    if (n, m) == (2, 4):
        meta = empty((rows, (k + 7) // 8), np.uint8, fill=255)
        vals2 = empty((rows, kc), np.uint16, fill=-1)
        S.nm_compress(xd, 2, 4, vals2, meta, S.NM_META_2BIT, None, k=k)
        sync()
        assert (host(meta, np.uint8) == O.pack_meta_2bit(i_ref)).all()
        assert (host(vals2, np.uint16) == v_ref).all()


# group widths of the (2N-2):2N weight family: no bitmask (groups straddle mask words)
SELECT_WIDE_CASES = [(4, 6), (1, 6), (6, 6), (8, 10), (3, 10), (10, 12), (6, 12), (12, 14), (7, 14), (13, 14)]


@pytest.mark.parametrize("n,m", SELECT_WIDE_CASES)
@pytest.mark.parametrize("rows,groups,pad", [(37, 131, 0), (5, 3, 2), (70, 64, 6)])
def test_select_bitexact_family_widths(n, m, rows, groups, pad):
    """S(X), values + u8 index and the scatter back, for m in {6, 10, 12, 14}; the
    bitmask is refused for these widths."""
    print(f"select wide n={n} m={m} rows={rows} groups={groups} pad={pad}", flush=True)
    rng = np.random.default_rng(2000 * m + n + rows)
    k = groups * m
    x = synth.student_t_bf16(rng, (rows, k), 4.0, 0.5)
    x[: min(4, rows)] = special_rows(k, rng)[: min(4, rows)]
    ld = k + pad
    xd = dev(x, ld)
    y = empty((rows, ld), np.uint16, fill=-1)
    S.nm_sparsify(xd, n, m, y, None, k=k)
    kc = k * n // m
    vals = empty((rows, kc), np.uint16, fill=-1)
    idx = empty((rows, kc), np.uint8, fill=255)
    S.nm_compress(xd, n, m, vals, idx, S.NM_META_U8, None, k=k)
    back = empty((rows, k), np.uint16, fill=-1)
    S.nm_decompress(vals, idx, S.NM_META_U8, rows, k, n, m, back)
    sync()
    s_ref, _ = O.sparsify(x, n, m)
    v_ref, i_ref = O.compress(x, n, m)
    assert (host(y, np.uint16)[:, :k] == s_ref).all()
    assert (host(y, np.uint16)[:, k:] == 0xFFFF).all()
    assert (host(vals, np.uint16) == v_ref).all()
    assert (host(idx, np.uint8) == i_ref).all()
    assert (host(back, np.uint16) == s_ref).all()
    mk = empty((rows, (k + 31) // 32), np.uint32)
    assert S.nm_sparsify(xd, n, m, y, mk, k=k, check=False) == S.NM_EUNSUPPORTED


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (2, 4)])
def test_select_full_size_sampled(n, m):
    """Down-projection activations at full size (8192 x 14336); oracle on one row of every
    128-row band; exactly n kept per group on every row."""
    print(f"select full n={n} m={m}", flush=True)
    d = synth.mlp_down_8of16(t_max=8192)
    x = d["x"]
    t, k = x.shape
    xd = dev(x)
    kc = k * n // m
    vals = empty((t, kc), np.uint16)
    idx = empty((t, kc), np.uint8)
    mask = empty((t, (k + 31) // 32), np.uint32)
    S.nm_compress(xd, n, m, vals, idx, S.NM_META_U8, mask)
    sync()
    rows = band_rows(t, 128, seed=n + m)
    v_ref, i_ref = O.compress(x[rows], n, m)
    keep = O.select_keep(x[rows], n, m)
    assert (host(vals, np.uint16)[rows] == v_ref).all()
    assert (host(idx, np.uint8)[rows] == i_ref).all()
    assert (host(mask, np.uint32)[rows] == O.pack_mask(keep)).all()
    # invariant on every row: exactly n kept per group
    pop = np.unpackbits(host(mask, np.uint32).view(np.uint8), axis=1, bitorder="little")
    assert (pop.reshape(t, -1, m).sum(-1) == n).all()


def scored_columns(rng, k, tiny=False):
    """Per-column fp32 weight magnitudes: L2 norms of a random W's columns, with repeated
    values, zeros and (tiny) subnormal-range products mixed in."""
    w = synth.normal_bf16(rng, (64, k), 0.02)
    c = np.sqrt((O.bf16_to_f64(w) ** 2).sum(0)).astype(np.float32)
    c[1::5] = c[0]
    c[3::17] = 0.0
    if tiny:
        c[::3] = np.float32(2.0 ** -110)
    return c


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (3, 8), (8, 16), (5, 16), (16, 32), (1, 32)])
@pytest.mark.parametrize("rows,groups,pad", [(37, 131, 0), (5, 3, 8), (70, 64, 16)])
def test_select_scored_bitexact(mode, n, m, rows, groups, pad):
    """Scored selection (weight magnitude alone, or activation weighted by it): S(X) and
    the bitmask bit for bit against the oracle, with ties in x and in the column scores,
    zero scores, products in the fp32 subnormal range and padded rows."""
    print(f"select scored mode={mode} n={n} m={m} rows={rows} groups={groups} pad={pad}", flush=True)
    rng = np.random.default_rng(3000 * m + 10 * n + rows + mode)
    k = groups * m
    x = synth.student_t_bf16(rng, (rows, k), 4.0, 0.5)
    x[: min(4, rows)] = special_rows(k, rng)[: min(4, rows)]
    x[~np.isfinite(O.bf16_to_f64(x))] = 0x3F80                 # scores need finite x (no inf, NaN)
    if rows > 5:
        x[5] = 0x0100                                           # tiny |x|: subnormal products
    c = scored_columns(rng, k, tiny=(rows == 37))
    ld = k + pad
    y = empty((rows, ld), np.uint16, fill=-1)
    words = (k + 31) // 32
    mask = empty((rows, words), np.uint32, fill=-1)
    S.nm_sparsify_scored(dev(x, ld), n, m, dev(c), mode, y, mask, k=k)
    sync()
    s_ref, keep = O.sparsify_scored(x, c, n, m, mode)
    assert (host(y, np.uint16)[:, :k] == s_ref).all()
    assert (host(y, np.uint16)[:, k:] == 0xFFFF).all()
    assert (host(mask, np.uint32) == O.pack_mask(keep)).all()


def test_select_scored_full_size_sampled():
    """Down-projection activations at full size (8192 x 14336), column scores = fp32 L2
    norms of the layer's W columns (activation weighted by weight magnitude); oracle on
    sampled rows, exactly n kept per group on every row."""
    print("select scored full", flush=True)
    d = synth.mlp_down_8of16(t_max=8192)
    x, w = d["x"], d["w"]
    t, k = x.shape
    c = np.sqrt((O.bf16_to_f64(w) ** 2).sum(0)).astype(np.float32)
    y = empty((t, k), np.uint16)
    mask = empty((t, (k + 31) // 32), np.uint32)
    S.nm_sparsify_scored(dev(x), 8, 16, dev(c), S.NM_SCORE_ACT_WEIGHTED, y, mask)
    sync()
    rows = band_rows(t, 128, seed=7)
    s_ref, keep = O.sparsify_scored(x[rows], c, 8, 16, O.SCORE_ACT_WEIGHTED)
    assert (host(y, np.uint16)[rows] == s_ref).all()
    assert (host(mask, np.uint32)[rows] == O.pack_mask(keep)).all()
    pop = np.unpackbits(host(mask, np.uint32).view(np.uint8), axis=1, bitorder="little")
    assert (pop.reshape(t, -1, 16).sum(-1) == 8).all()


def test_select_deterministic():
    rng = np.random.default_rng(5)
    x = synth.student_t_bf16(rng, (256, 4096), 4.0, 1.0)
    xd = dev(x)
    outs = []
    for _ in range(10):
        v = empty((256, 2048), np.uint16)
        i = empty((256, 2048), np.uint8)
        S.nm_compress(xd, 8, 16, v, i, S.NM_META_U8)
        sync()
        outs.append((host(v, np.uint16).copy(), host(i, np.uint8).copy()))
    for v, i in outs[1:]:
        assert (v == outs[0][0]).all() and (i == outs[0][1]).all()


@pytest.mark.parametrize("n,m,fmt", [(2, 4, 1), (2, 4, 0), (8, 16, 0), (16, 32, 0), (6, 8, 0), (3, 8, 0)])
def test_decompress_roundtrip(n, m, fmt):
    rng = np.random.default_rng(77 + m)
    rows, k = 29, m * 45
    x = synth.normal_bf16(rng, (rows, k))
    v_ref, i_ref = O.compress(x, n, m)
    meta = O.pack_meta_2bit(i_ref) if fmt == 1 else i_ref
    y = empty((rows, k), np.uint16, fill=-1)
    S.nm_decompress(dev(v_ref), dev(meta), fmt, rows, k, n, m, y)
    sync()
    assert (host(y, np.uint16) == O.decompress(v_ref, i_ref, n, m, k)).all()


# ---------------------------------------------------------------------- slide ---

@pytest.mark.parametrize("ns", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("fmt", [0, 1])
def test_lower_slide_bitexact(ns, fmt):
    rng = np.random.default_rng(ns * 10 + fmt)
    m, n = 2 * ns, 2 * ns - 2
    rows, k = 23, 2 * ns * 37
    w = synth.normal_bf16(rng, (rows, k), 0.02)
    w[0, :m] = 0x3F80                                 # a fully tied group
    v, i = O.compress(w, n, m)
    vp_ref, ip_ref = O.slide_lower(v, i, k, ns)
    kp = O.lowered_k(k, ns)
    vo = empty((rows, kp // 2), np.uint16, fill=-1)
    mo = empty((rows, kp // 2 if fmt == 0 else (kp + 7) // 8), np.uint8, fill=255)
    S.nm_lower_slide(dev(v), dev(i), rows, k, ns, vo, mo, fmt)
    sync()
    assert (host(vo, np.uint16) == vp_ref).all()
    want = ip_ref if fmt == 0 else O.pack_meta_2bit(ip_ref)
    assert (host(mo, np.uint8) == want).all()


@pytest.mark.parametrize("ns", [2, 4, 6])
def test_lift_bitexact(ns):
    rng = np.random.default_rng(ns)
    t, k = 19, 2 * ns * 21
    x = synth.normal_bf16(rng, (t, k))
    kp = O.lowered_k(k, ns)
    xo = empty((t, kp + 8), np.uint16, fill=-1)
    S.nm_slide_lift(dev(x), ns, xo, k=k, ldo=kp + 8)
    sync()
    assert (host(xo, np.uint16)[:, :kp] == O.lift(x, ns)).all()


# -------------------------------------------------------------- activation spmm ---

def run_act(x, w, n, m, route=None, w8=None, s8=None, workspace=True, accumulate=0, y0=None, want_mask=True):
    t, k = x.shape
    o = w.shape[0] if w is not None else w8.shape[0]
    xd = dev(x)
    if w8 is not None:
        wd_, dtype, sd = dev(w8), S.NM_W_FP8E4M3, dev(s8)
    else:
        wd_, dtype, sd = dev(w), S.NM_W_BF16, None
    y = dev(y0.astype(np.float32)) if y0 is not None else empty((t, o), np.float32, fill=float("nan"))
    mask = empty((t, (k + 31) // 32), np.uint32, fill=-1) if want_mask else None
    a = mk_args(S.NM_ACT_DYNAMIC, t, o, k, xd, wd_, y, n=n, m=m, w_dtype=dtype, w_scale=sd,
                x_mask_out=mask, accumulate=accumulate, route=S.route_bits("act_" + route) if route else 0)
    ws = None
    if workspace:
        nb = S.nm_spmm_workspace_size(a)
        ws = empty((max(nb, 16),), np.uint8)
        a.workspace, a.workspace_bytes = ws.data_ptr(), nb
    spmm_call(a)
    sync()
    return host(y, np.float32), (host(mask, np.uint32) if mask is not None else None)


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (4, 8), (2, 4), (1, 4), (6, 8)])
@pytest.mark.parametrize("route", ["fused", "mask", "sx", "sparse_x"])
@pytest.mark.parametrize("t,o,k", [(300, 200, 1024), (17, 520, 1056), (513, 264, 2048)])
def test_spmm_act_dynamic(n, m, route, t, o, k):
    print(f"spmm act n={n} m={m} route={route} t={t} o={o} k={k}", flush=True)
    if k % m:
        pytest.skip("k not a multiple of m")
    rng = np.random.default_rng(t + o + k + m)
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    y, mask = run_act(x, w, n, m, route=route)
    sx, keep = O.sparsify(x, n, m)
    assert (mask == O.pack_mask(keep)).all()
    check_gemm(y, O.gemm(sx, w), sx, w, label=f"act {n}:{m} {route}")


@pytest.mark.parametrize("kernel", ["lds", "regs"])
@pytest.mark.parametrize("t,o,k", [(1000, 600, 1024), (257, 300, 640), (64, 2000, 2048)])
def test_spmm_act_masked_kernels(kernel, t, o, k):
    """Two-pass route (nm_sparsify mask + ACT_MASKED) on both product kernels, ragged
    tiles in T and O."""
    print(f"masked kernel={kernel} t={t} o={o} k={k}", flush=True)
    rng = np.random.default_rng(t + o)
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    xd, wdv = dev(x), dev(w)
    mask = empty((t, k // 32), np.uint32)
    S.nm_sparsify(xd, 8, 16, None, mask)
    y = empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(S.NM_ACT_MASKED, t, o, k, xd, wdv, y, n=8, m=16, x_meta=mask, route=S.route_bits("tile_" + kernel))
    spmm_call(a)
    sync()
    assert f"tile_{kernel}" in taken() and "mask" in taken()
    sx, keep = O.sparsify(x, 8, 16)
    assert (host(mask, np.uint32) == O.pack_mask(keep)).all()
    check_gemm(host(y, np.float32), O.gemm(sx, w), sx, w, label=f"masked {kernel}")
    # the same kernel with X already sparsified (no mask)
    y2 = empty((t, o), np.float32, fill=float("nan"))
    sxd = dev(sx)
    a2 = mk_args(S.NM_ACT_MASKED, t, o, k, sxd, wdv, y2, n=8, m=16, x_meta=mask,
                 route=S.route_bits("tile_" + kernel))
    spmm_call(a2)
    sync()
    check_gemm(host(y2, np.float32), O.gemm(sx, w), sx, w, label=f"masked presparsified {kernel}")
    # x already S(X), no mask: the plain product
    y3 = empty((t, o), np.float32, fill=float("nan"))
    a3 = mk_args(S.NM_ACT_MASKED, t, o, k, sxd, wdv, y3, n=8, m=16)
    nb = S.nm_spmm_workspace_size(a3)
    ws3 = empty((max(nb, 16),), np.uint8)
    a3.workspace, a3.workspace_bytes = ws3.data_ptr(), nb
    with use_route("tile_" + kernel):
        a3.route = _ROUTE["route"]
        spmm_call(a3)
        sync()
    check_gemm(host(y3, np.float32), O.gemm(sx, w), sx, w, label=f"S(X) no mask {kernel}")


def test_spmm_act_2of4_layer():
    """Single 2:4 activation-sparse layer (X 64x512, W 512x512): the weight-streaming
    few-token kernel, and with the no_few hint the S(X) product (workspace), the fused
    dense path (none) and, under the act_sparse_x hint, the sparse matrix path (compress +
    SMFMAC with X as the sparse operand)."""
    d = synth.layer_2of4_small()
    x, w = d["x"], d["w"]
    sx, keep = O.sparsify(x, 2, 4)
    ref = O.gemm(sx, w)
    for hints in ((), ("no_few",), ("no_few", "act_sparse_x")):
        for ws in (True, False):
            with use_route(*hints):
                y, mask = run_act(x, w, 2, 4, workspace=ws)
                if "act_sparse_x" in hints and ws:
                    assert "sparse_mma" in taken(), taken()
            assert (mask == O.pack_mask(keep)).all()
            check_gemm(y, ref, sx, w, label=f"2:4 layer ws={ws} hints={hints}")


# route hints of the few-token dispatch: weight-streaming kernel, split-K tile kernel
# (K % 64 == 0; others fall back to streaming) with its default and forced workgroup
# counts, or the large-T tile kernels
FEW_ROUTES = {"stream": (("few_stream",), {}), "tile": (("few_tile",), {}),
              "tile_wg37": (("few_tile",), {"tile_wg": 37}), "tile_wg100": (("few_tile",), {"tile_wg": 100}),
              "off": (("no_few",), {})}


def run_w(mode, x, v, mt, o, k, ns=2, workspace=True, accumulate=0, y0=None):
    t = x.shape[0]
    y = dev(y0.astype(np.float32)) if y0 is not None else empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(mode, t, o, k, dev(x), v, y, ns=ns, w_meta=mt, w_meta_fmt=S.NM_META_2BIT,
                accumulate=accumulate)
    ws = None
    if workspace:
        nb = S.nm_spmm_workspace_size(a)
        ws = empty((max(nb, 16),), np.uint8)
        a.workspace, a.workspace_bytes = ws.data_ptr(), nb
    spmm_call(a)
    sync()
    return host(y, np.float32)


@pytest.mark.parametrize("route", list(FEW_ROUTES))
@pytest.mark.parametrize("t", [1, 7, 16, 33, 64, 100, 128])
@pytest.mark.parametrize("k", [1056, 1024])
def test_few_token_kernels(route, t, k):
    """Few-token shapes on each route: 8:16 activations (bf16 and fp8 weights), 2:4 and
    6:8-lowered weights, ragged O (200 rows: the reduction is also split across
    workgroups and summed by the second pass), with and without a workspace."""
    print(f"few-token t={t} k={k} route={route}", flush=True)
    rng = np.random.default_rng(t)
    o = 200
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    names, tune = FEW_ROUTES[route]
    with use_route(*names, **tune):
        sx, _ = O.sparsify(x, 8, 16)
        for ws in (True, False):
            y, _ = run_act(x, w, 8, 16, workspace=ws)
            check_gemm(y, O.gemm(sx, w), sx, w, label=f"8:16 bf16 ws={ws}")
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        y8, _ = run_act(x, None, 8, 16, w8=q, s8=sc)
        wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
        check_gemm(y8, O.spmm_act_fp8(x, q, sc, 8, 16), sx, wdeq, label="8:16 fp8")
        v, mt = gpu_compress_2of4(w)
        ws24, _ = O.sparsify(w, 2, 4)
        for ws in (True, False):
            yw = run_w(S.NM_W_COMPRESSED, x, v, mt, o, k, workspace=ws)
            check_gemm(yw, O.gemm(x, ws24), x, ws24, label=f"w 2:4 ws={ws}")
        k8 = 1024
        x8 = np.ascontiguousarray(x[:, :k8])
        vp, mp = slide_pack_gpu(np.ascontiguousarray(w[:, :k8]), 4)
        ys = run_w(S.NM_W_SLIDE, x8, vp, mp, o, k8, ns=4)
        pr, _ = O.sparsify(np.ascontiguousarray(w[:, :k8]), 6, 8)
        check_gemm(ys, O.gemm(x8, pr), x8, pr, label="slide 6:8")


@pytest.mark.parametrize("wg", [1, 6])
@pytest.mark.parametrize("t", [40, 100])
@pytest.mark.parametrize("nsteps", [1, 2, 3, 4, 5, 6, 7, 9])
def test_few_token_tile_step_counts(nsteps, t, wg):
    """The split-K tile kernels' multi-stage K-loop at every short step count: K = 64
    nsteps, with tile_wg = 1 (no split: each workgroup runs all nsteps K-steps) and 6
    (three splits of the two o-tiles), covering every remainder of the steps modulo the
    stage count, the re-requested last step, and the one-step case.  Dense weights with
    8:16 activations, 2:4 weights, and the hybrid (sparse then dense K-steps)."""
    print(f"tile steps={nsteps} t={t} wg={wg}", flush=True)
    rng = np.random.default_rng(100 * nsteps + t + wg)
    o, k = 200, 64 * nsteps
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    with use_route("few_tile", tile_wg=wg):
        sx, _ = O.sparsify(x, 8, 16)
        y, _ = run_act(x, w, 8, 16)
        assert "tile_lds" in taken(), taken()
        check_gemm(y, O.gemm(sx, w), sx, w, label=f"8:16 steps={nsteps}")
        v, mt = gpu_compress_2of4(w)
        ws24, _ = O.sparsify(w, 2, 4)
        yw = run_w(S.NM_W_COMPRESSED, x, v, mt, o, k)
        assert "tile_lds" in taken() and "sparse_mma" in taken(), taken()
        check_gemm(yw, O.gemm(x, ws24), x, ws24, label=f"w 2:4 steps={nsteps}")
        if nsteps >= 2:
            # hybrid: the first 64 (nsteps - 1) columns sparse, the last 64 dense
            ks, kd = 64 * (nsteps - 1), 64
            wsp, _ = O.sparsify(np.ascontiguousarray(w[:, :ks]), 2, 4)
            vs, ms = gpu_compress_2of4(np.ascontiguousarray(w[:, :ks]))
            wd = np.ascontiguousarray(w[:, ks:])
            yh = run_hybrid(x, None, ks, None, kd, vs, ms, dev(wd), o)
            ref = O.gemm(np.ascontiguousarray(x[:, :ks]), wsp) + O.gemm(np.ascontiguousarray(x[:, ks:]), wd)
            wcat = np.concatenate([wsp, wd], axis=1)
            check_gemm(yh, ref, x, wcat, label=f"hybrid steps={nsteps}")


@pytest.mark.parametrize("wpb,splits", [(4, 0), (8, 0), (16, 0), (16, 3), (4, 7)])
@pytest.mark.parametrize("t", [1, 20, 70])
def test_few_token_partition_overrides(wpb, splits, t):
    """The weight-streaming kernel under forced in-workgroup wave counts and cross-
    workgroup splits (every partition of the reduction must give the same result up to
    rounding), with accumulation into a nonzero Y; then bitwise determinism of a repeat
    call.  O = 64 (few row blocks), K = 4096."""
    print(f"few-token partition wpb={wpb} splits={splits} t={t}", flush=True)
    rng = np.random.default_rng(7 * t + wpb)
    o, k = 64, 4096
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    with use_route("few_stream", few_wpb=wpb, few_splits=splits):
        sx, _ = O.sparsify(x, 8, 16)
        y, _ = run_act(x, w, 8, 16, accumulate=1, y0=y0)
        check_gemm(y - y0, O.gemm(sx, w), sx, w, label="8:16 accumulate")
        y_again, _ = run_act(x, w, 8, 16, accumulate=1, y0=y0)
        assert (y.view(np.uint32) == y_again.view(np.uint32)).all(), "repeat call differs"
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        y8, _ = run_act(x, None, 8, 16, w8=q, s8=sc)
        wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
        check_gemm(y8, O.spmm_act_fp8(x, q, sc, 8, 16), sx, wdeq, label="8:16 fp8")
        v, mt = gpu_compress_2of4(w)
        ws24, _ = O.sparsify(w, 2, 4)
        yw = run_w(S.NM_W_COMPRESSED, x, v, mt, o, k, accumulate=1, y0=y0)
        check_gemm(yw - y0, O.gemm(x, ws24), x, ws24, label="w 2:4 accumulate")
        vp, mp = slide_pack_gpu(w, 4)
        ys = run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=4)
        pr, _ = O.sparsify(w, 6, 8)
        check_gemm(ys, O.gemm(x, pr), x, pr, label="slide 6:8")
        sc_, dc_, wv, wm, wdd = hybrid_pack_gpu(w, 1024)
        sync()
        sp, de, hv, hi, hwd = O.hybrid_pack(w, 1024)
        wh = w.copy()
        wh[:, sp] = O.decompress(hv, hi, 2, 4, k - 1024)
        yh = run_hybrid(x, sc_, k - 1024, dc_, 1024, wv, wm, wdd, o)
        check_gemm(yh, O.hybrid_gemm(x, sp, de, hv, hi, hwd), x, wh, label="hybrid")


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32), (2, 4), (4, 8), (1, 4), (31, 32)])
@pytest.mark.parametrize("k,o", [(1056, 264), (4128, 1024), (96, 8)])
def test_single_token_kmajor_gather(n, m, k, o):
    """One token with K-major weights: only the kept K-rows are read.  Result, mask and
    accumulation against the oracle; the route needs o % 8 == 0 and a workspace."""
    if k % m:
        pytest.skip("k not a multiple of m")
    print(f"gather n={n} m={m} k={k} o={o}", flush=True)
    rng = np.random.default_rng(k + o + m)
    x = synth.student_t_bf16(rng, (1, k), 4.0, 0.5)
    x[0, :4] = np.array([0x3F80, 0x3F80, 0xBF80, 0x0000], np.uint16)     # ties
    w = synth.normal_bf16(rng, (o, k), 0.02)
    wk = dev(np.ascontiguousarray(w.T))
    sx, keep = O.sparsify(x, n, m)
    ref = O.gemm(sx, w)
    y0 = rng.standard_normal((1, o)).astype(np.float32)
    for acc in (0, 1):
        y = dev(y0) if acc else empty((1, o), np.float32, fill=float("nan"))
        mask = empty((1, (k + 31) // 32), np.uint32, fill=-1)
        a = mk_args(S.NM_ACT_DYNAMIC, 1, o, k, dev(x), dev(w), y, n=n, m=m, w_kmajor=wk,
                             x_mask_out=mask, accumulate=acc)
        nb = S.nm_spmm_workspace_size(a)
        assert nb > 0 and nb < 1 << 24          # partial sums only
        ws = empty((nb,), np.uint8)
        a.workspace, a.workspace_bytes = ws.data_ptr(), nb
        S.nm_spmm(a)
        sync()
        got = host(y, np.float32)
        check_gemm(got - (y0 if acc else 0), ref, sx, w, label=f"gather acc={acc}")
        assert (host(mask, np.uint32) == O.pack_mask(keep)).all()
        if acc == 0:   # repeat: bitwise identical
            S.nm_spmm(a)
            sync()
            assert (host(y, np.float32).view(np.uint32) == got.view(np.uint32)).all()


def test_single_token_kmajor_full_size():
    """8:16 down-projection, one token, K-major weights 14336 x 4096."""
    d = synth.mlp_down_8of16(t_max=1)
    x, w = d["x"], d["w"]
    o, k = w.shape
    wk = dev(np.ascontiguousarray(w.T))
    y = empty((1, o), np.float32, fill=float("nan"))
    a = mk_args(S.NM_ACT_DYNAMIC, 1, o, k, dev(x), dev(w), y, n=8, m=16, w_kmajor=wk)
    nb = S.nm_spmm_workspace_size(a)
    ws = empty((nb,), np.uint8)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nb
    S.nm_spmm(a)
    sync()
    sx, _ = O.sparsify(x, 8, 16)
    check_gemm(host(y, np.float32), O.gemm(sx, w), sx, w, label="gather full")


def test_spmm_act_compressed_2of4_and_8of16():
    rng = np.random.default_rng(9)
    for n, m, fmt in [(2, 4, 1), (8, 16, 0), (2, 4, 0)]:
        t, o, k = 150, 272, 512
        x = synth.normal_bf16(rng, (t, k))
        w = synth.normal_bf16(rng, (o, k), 0.02)
        v, i = O.compress(x, n, m)
        meta = O.pack_meta_2bit(i) if fmt == 1 else i
        y = empty((t, o), np.float32, fill=float("nan"))
        a = mk_args(S.NM_ACT_COMPRESSED, t, o, k, dev(v), dev(w), y, n=n, m=m, x_meta=dev(meta),
                             x_meta_fmt=fmt, ldx=0)
        nb = S.nm_spmm_workspace_size(a)
        ws = empty((nb,), np.uint8)
        a.workspace, a.workspace_bytes = ws.data_ptr(), nb
        S.nm_spmm(a)
        sync()
        sx, _ = O.sparsify(x, n, m)
        check_gemm(host(y, np.float32), O.gemm(sx, w), sx, w, label=f"compressed {n}:{m} fmt={fmt}")


def test_spmm_act_accumulate_and_fp8():
    rng = np.random.default_rng(11)
    t, o, k = 96, 384, 2048
    x = synth.student_t_bf16(rng, (t, k), 4.0, 1.0)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    q, s = synth.fp8_e4m3_quantize_rows(w)
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    for route in ("fused", "mask", "sx"):
        y, _ = run_act(x, None, 16, 32, route=route, w8=q, s8=s)
        sx, _ = O.sparsify(x, 16, 32)
        wdeq = O.fp8_e4m3_to_f64(q) * s[:, None].astype(np.float64)
        check_gemm(y, O.spmm_act_fp8(x, q, s, 16, 32), sx, wdeq, label=f"fp8 {route}")
        y2, _ = run_act(x, w, 8, 16, route=route, accumulate=1, y0=y0)
        sx, _ = O.sparsify(x, 8, 16)
        check_gemm(y2 - y0, O.gemm(sx, w), sx, w, label=f"accumulate {route}")


@pytest.mark.parametrize("widen", [False, True])
@pytest.mark.parametrize("t,o,k", [(600, 300, 1024), (520, 136, 1056), (1030, 520, 2048)])
def test_spmm_act_fp8_large_tokens(t, o, k, widen):
    """fp8 weights at prefill sizes (K % 64 == 0): codes staged straight into LDS and
    widened per fragment, or (the fp8_widen hint) widened once to bf16 in the workspace;
    otherwise the register-staged fp8 kernel.  Scale, accumulate, ragged tiles."""
    print(f"fp8 large t={t} o={o} k={k} widen={widen}", flush=True)
    rng = np.random.default_rng(t + k)
    x = synth.student_t_bf16(rng, (t, k), 4.0, 1.0)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    q, sc = synth.fp8_e4m3_quantize_rows(w)
    wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    with use_route(*(("fp8_widen",) if widen else ())):
        for n, m in ((16, 32), (8, 16)):
            sx, keep = O.sparsify(x, n, m)
            ref = O.spmm_act_fp8(x, q, sc, n, m)
            y, mask = run_act(x, None, n, m, w8=q, s8=sc)
            assert (mask == O.pack_mask(keep)).all()
            check_gemm(y, ref, sx, wdeq, label=f"fp8 {n}:{m}")
            y2, _ = run_act(x, None, n, m, w8=q, s8=sc, accumulate=1, y0=y0)
            check_gemm(y2 - y0, ref, sx, wdeq, label=f"fp8 {n}:{m} accumulate")


def test_fp8_decode_all_codes():
    """Every finite e4m3 code through the fp8 weight loader equals the oracle's decode."""
    codes = np.arange(256, dtype=np.uint8)
    codes[np.isnan(O.fp8_e4m3_to_f64(codes))] = 0                 # the two NaN codes -> +0
    k = 256
    w8 = np.zeros((len(codes), k), np.uint8)
    w8[:, 5] = codes                                               # one code per row, column 5
    x = np.zeros((1, k), np.uint16)
    x[0, :] = 0x3F80                                               # all ones: 8:16 keeps the first 8
    y, _ = run_act(x, None, 8, 16, route="fused", w8=w8, s8=np.ones(len(codes), np.float32))
    assert (y[0].astype(np.float64) == O.fp8_e4m3_to_f64(codes)).all()


LAYER_GROUPS = {"q": ("q",), "k": ("k",), "v": ("v",), "o": ("o",), "gate": ("gate",), "up": ("up",),
                "down": ("down",), "qkv": ("q", "k", "v"), "gate_up": ("gate", "up")}


@pytest.fixture(scope="module")
def layer8b():
    return synth.transformer_layer(t_max=8192, with_fp8=True)


@pytest.mark.parametrize("t", [64, 8192])
@pytest.mark.parametrize("group", list(LAYER_GROUPS))
def test_layer_full_size_sampled(layer8b, group, t):
    """The 8B-shaped layer's linears at full size, each alone and with the linears that
    share an input concatenated along the output dimension (q|k|v 6144 x 4096, gate|up
    28672 x 4096), as the layer measurement runs them: 16:32 and 8:16 activations, bf16
    and fp8 weights, workspace from the size query.  Every output written; the oracle on
    one row of every 256-row band (every 8-row band at 64 tokens)."""
    import torch

    parts = LAYER_GROUPS[group]
    print(f"layer {group} t={t}", flush=True)
    st = synth.TRANSFORMER_SHAPES[parts[0]][2]
    x = layer8b["x"][st][:t]
    w = np.concatenate([layer8b["w"][p] for p in parts], 0)
    w8 = np.concatenate([layer8b["w8"][p] for p in parts], 0)
    s8 = np.concatenate([layer8b["s8"][p] for p in parts], 0)
    o, k = w.shape
    rows = band_rows(t, 256 if t > 256 else 8, seed=t + o)
    xd = dev(x)
    wdeq = O.fp8_e4m3_to_f64(w8) * s8[:, None].astype(np.float64)
    for (n, m) in ((16, 32), (8, 16)):
        sx, keep = O.sparsify(x[rows], n, m)
        for kind in ("bf16", "fp8"):
            y = torch.full((t, o), float("nan"), dtype=torch.float32, device="cuda")
            if kind == "bf16":
                a = mk_args(S.NM_ACT_DYNAMIC, t, o, k, xd, dev(w), y, n=n, m=m)
            else:
                a = mk_args(S.NM_ACT_DYNAMIC, t, o, k, xd, dev(w8), y, n=n, m=m,
                                     w_dtype=S.NM_W_FP8E4M3, w_scale=dev(s8))
            nb = S.nm_spmm_workspace_size(a)
            ws = empty((max(nb, 16),), np.uint8)
            a.workspace, a.workspace_bytes = ws.data_ptr(), nb
            S.nm_spmm(a)
            sync()
            check_all_written(y, f"layer {group} t={t} {n}:{m} {kind}")
            yr = y[torch.from_numpy(rows).cuda()].cpu().numpy()
            if kind == "bf16":
                check_gemm(yr, O.gemm(sx, w), sx, w, label=f"layer {group} t={t} {n}:{m} bf16")
            else:
                check_gemm(yr, O.spmm_act_fp8(x[rows], w8, s8, n, m), sx, wdeq,
                           label=f"layer {group} t={t} {n}:{m} fp8")
            del y, ws, a


@pytest.fixture(scope="module")
def down_full():
    """The 8:16 down-projection workload at full size with the oracle's selection of every
    row (computed once per module)."""
    d = synth.mlp_down_8of16(t_max=8192)
    sx_all, keep_all = O.sparsify(d["x"], 8, 16)
    return d["x"], d["w"], sx_all, O.pack_mask(keep_all)


@pytest.mark.parametrize("route", ["fused", "mask", "sx"])
def test_spmm_act_full_size_sampled(route, down_full):
    """8:16 down-projection at 300 (the split tile kernel on the default route), 2048 and
    8192 tokens: the mask of every row bit-exact, every output written, random projections
    of the whole output, and the oracle on one row of every 128-row band."""
    print(f"act full route={route}", flush=True)
    x_all, w, sx_all, mask_all = down_full
    wv = O.bf16_to_f64(w)
    for t in (300, 2048, 8192):
        x = x_all[:t]
        y, mask = run_act(x, w, 8, 16, route=route)
        assert (mask == mask_all[:t]).all()
        assert np.isfinite(y).all(), f"full t={t}: unwritten outputs"
        check_projection(y, O.bf16_to_f64(sx_all[:t]), wv, label=f"full t={t} projection")
        rows = band_rows(t, 128, seed=t)
        sx = sx_all[rows]
        check_gemm(y[rows], O.gemm(sx, w), sx, w, label=f"full t={t}")


@pytest.mark.parametrize("t", [1, 16, 33, 64, 128])
def test_spmm_act_decode_full_size_sampled(t):
    """8:16 down-projection (W 4096 x 14336) at decode token counts on the default routes
    (select + streaming kernel up to 32 tokens, select + split-K tile kernel above);
    the oracle on every output row."""
    print(f"act decode full t={t}", flush=True)
    d = synth.mlp_down_8of16(t_max=128)
    x, w = d["x"][:t], d["w"]
    y, mask = run_act(x, w, 8, 16)
    sx, keep = O.sparsify(x, 8, 16)
    assert (mask == O.pack_mask(keep)).all()
    check_gemm(y, O.gemm(sx, w), sx, w, label=f"decode full t={t}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("t", [2, 7, 16, 17, 32])
def test_few_token_blocked_sx(t, kind):
    """2-32 tokens on the weight-streaming kernel: S(X) staged in 16-token blocks (each
    32-position piece of a block's rows contiguous) against the row-major staging (the
    row_sx hint): the same bits and the same selection mask, and the oracle on every row.
    Ragged token blocks (7, 17 tokens), ragged 16-row weight blocks, and a reduction length
    whose parts end unevenly (the checked tail loads)."""
    print(f"blocked S(X) t={t} {kind}", flush=True)
    rng = np.random.default_rng(t * 3 + len(kind))
    o, k = 520, 4064
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    kw = {}
    if kind == "fp8":
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        kw = dict(w8=q, s8=sc)
    wa = None if kind == "fp8" else w
    y, mask = run_act(x, wa, 8, 16, **kw)
    tk = taken()
    assert {"select", "few_stream"} <= tk, tk
    with use_route("row_sx"):
        y_row, mask_row = run_act(x, wa, 8, 16, **kw)
    assert np.array_equal(y.view(np.uint32), y_row.view(np.uint32)), "blocked vs row-major S(X)"
    assert (mask == mask_row).all()
    sx, keep = O.sparsify(x, 8, 16)
    assert (mask == O.pack_mask(keep)).all()
    if kind == "bf16":
        check_gemm(y, O.gemm(sx, w), sx, w, label=f"blocked S(X) t={t}")
    else:
        wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
        check_gemm(y, O.spmm_act_fp8(x, q, sc, 8, 16), sx, wdeq, label=f"blocked S(X) fp8 t={t}")


@pytest.mark.parametrize("t", [16, 64, 128])
def test_spmm_act_fp8_decode_full_size_sampled(t):
    """fp8 weights (per-row scales) on the 8:16 down-projection (W 4096 x 14336) at decode
    token counts; the oracle on every output row."""
    print(f"fp8 decode full t={t}", flush=True)
    d = synth.mlp_down_8of16(t_max=128)
    x, w = d["x"][:t], d["w"]
    q, sc = synth.fp8_e4m3_quantize_rows(w)
    y, mask = run_act(x, None, 8, 16, w8=q, s8=sc)
    sx, keep = O.sparsify(x, 8, 16)
    assert (mask == O.pack_mask(keep)).all()
    wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    check_gemm(y, O.spmm_act_fp8(x, q, sc, 8, 16), sx, wdeq, label=f"fp8 decode full t={t}")


# ------------------------------------------------------------------- weight 2:4 ---

def gpu_compress_2of4(w):
    o, k = w.shape
    v = empty((o, k // 2), np.uint16)
    mt = empty((o, (k + 7) // 8), np.uint8)
    S.nm_compress(dev(w), 2, 4, v, mt, S.NM_META_2BIT)
    return v, mt


@pytest.mark.parametrize("t,o,k", [(77, 300, 512), (256, 256, 1024), (5, 33, 96)])
def test_spmm_w_compressed(t, o, k):
    rng = np.random.default_rng(t * o)
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    v, mt = gpu_compress_2of4(w)
    y = empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(S.NM_W_COMPRESSED, t, o, k, dev(x), v, y, w_meta=mt, w_meta_fmt=S.NM_META_2BIT)
    S.nm_spmm(a)
    sync()
    ws, _ = O.sparsify(w, 2, 4)
    check_gemm(host(y, np.float32), O.gemm(x, ws), x, ws, label="w 2:4")


def slide_pack_gpu(w, ns):
    o, k = w.shape
    n, m = 2 * ns - 2, 2 * ns
    v = empty((o, k * n // m), np.uint16)
    i = empty((o, k * n // m), np.uint8)
    S.nm_compress(dev(w), n, m, v, i, S.NM_META_U8)
    kp = O.lowered_k(k, ns)
    vp = empty((o, kp // 2), np.uint16)
    mp = empty((o, (kp + 7) // 8), np.uint8)
    S.nm_lower_slide(v, i, o, k, ns, vp, mp, S.NM_META_2BIT)
    return vp, mp


@pytest.mark.parametrize("ns", [4, 2, 8])
@pytest.mark.parametrize("t", [1, 16, 130, 300])
def test_spmm_w_slide(ns, t):
    print(f"slide ns={ns} t={t}", flush=True)
    rng = np.random.default_rng(ns * 1000 + t)
    o, k = 264, 2 * ns * 40
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    vp, mp = slide_pack_gpu(w, ns)
    sync()
    pruned, _ = O.sparsify(w, 2 * ns - 2, 2 * ns)
    v, i = O.compress(w, 2 * ns - 2, 2 * ns)
    vp_ref, ip_ref = O.slide_lower(v, i, k, ns)
    assert (host(vp, np.uint16) == vp_ref).all()
    assert (host(mp, np.uint8) == O.pack_meta_2bit(ip_ref)).all()
    y = empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(S.NM_W_SLIDE, t, o, k, dev(x), vp, y, ns=ns, w_meta=mp, w_meta_fmt=S.NM_META_2BIT)
    S.nm_spmm(a)
    sync()
    # the lowered product must equal the dense product on the same pruned W
    check_gemm(host(y, np.float32), O.gemm(x, pruned), x, pruned, label=f"slide ns={ns}")


@pytest.mark.parametrize("ns", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("t,o,hint", [(40, 2056, "few_tile"), (100, 2056, "few_tile"), (300, 264, "tile_lds"),
                                      (1030, 1040, "tile_lds")])
def test_slide_lift_in_loads_bitexact(ns, t, o, hint):
    """Lowered (2N-2):2N weights on the direct-to-LDS tile kernels: the loads build the
    lifted X rows from the raw X (no lifted copy), so the stages hold the same bytes as
    when X is lifted into the workspace first (the lift_copy hint): the same bits, and
    the dense product on the pruned W within tolerance.  Few-token split tiles (40 and 100
    tokens, 2056 rows) and the large-token kernel (ragged tiles in both dimensions)."""
    print(f"slide lift in loads ns={ns} t={t} o={o}", flush=True)
    rng = np.random.default_rng(ns * 7 + t)
    k = 2 * ns * 64 * (3 if ns != 8 else 1)
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    vp, mp = slide_pack_gpu(w, ns)
    pruned, _ = O.sparsify(w, 2 * ns - 2, 2 * ns)
    hints = (hint,) if hint else ()
    with use_route(*hints):
        y = run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=ns)
        assert "tile_lds" in taken() and "lift" not in taken(), taken()
        with use_route("lift_copy"):
            y_copy = run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=ns)
            assert "tile_lds" in taken() and "lift" in taken(), taken()
    assert np.array_equal(y.view(np.uint32), y_copy.view(np.uint32)), "lift in loads vs lifted copy"
    check_gemm(y, O.gemm(x, pruned), x, pruned, label=f"slide ns={ns} t={t} lift in loads")


@pytest.mark.parametrize("ns", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("t,o,groups", [(2, 264, 48), (7, 520, 200), (16, 4096, 512), (29, 264, 72)])
def test_stream_lift_pairs_bitexact(ns, t, o, groups):
    """Lowered (2N-2):2N weights on the few-token weight-streaming kernel with X in global
    memory: its whole-stage loads take each pair of lifted windows with one 16-byte load
    of the raw row (starting a dword early where the load would pass the row end), the
    ragged end window by window.  The same bits as the same kernel on X lifted beforehand
    (plain loads of the lifted row, W_COMPRESSED over K'), and the dense product on the
    pruned W within tolerance.  Row lengths with whole stages only and with ragged ends."""
    print(f"stream lift pairs ns={ns} t={t} o={o} groups={groups}", flush=True)
    rng = np.random.default_rng(ns * 31 + t)
    k = 2 * ns * groups
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    vp, mp = slide_pack_gpu(w, ns)
    kp = O.lowered_k(k, ns)
    with use_route("few_stream"):
        y = run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=ns)
        assert "few_stream" in taken() and "tile_lds" not in taken(), taken()
        y_pre = run_w(S.NM_W_COMPRESSED, O.lift(x, ns), vp, mp, o, kp)
        assert "few_stream" in taken(), taken()
    assert np.array_equal(y.view(np.uint32), y_pre.view(np.uint32)), "lifted loads vs pre-lifted X"
    pruned, _ = O.sparsify(w, 2 * ns - 2, 2 * ns)
    check_gemm(y, O.gemm(x, pruned), x, pruned, label=f"stream lift pairs ns={ns} t={t}")


@pytest.mark.parametrize("ns", [3, 5, 6, 7])
def test_spmm_w_slide_odd_family(ns):
    """4:6, 8:10, 10:12 and 12:14 weights end to end on the GPU: compressed by the
    library (bit-exact against the oracle), lowered and multiplied."""
    rng = np.random.default_rng(ns)
    t, o, k = 70, 136, 2 * ns * 24
    x = synth.normal_bf16(rng, (t, k))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    v_ref, i_ref = O.compress(w, 2 * ns - 2, 2 * ns)
    v = empty(v_ref.shape, np.uint16)
    i = empty(i_ref.shape, np.uint8)
    S.nm_compress(dev(w), 2 * ns - 2, 2 * ns, v, i, S.NM_META_U8, None)
    sync()
    assert (host(v, np.uint16) == v_ref).all()
    assert (host(i, np.uint8) == i_ref).all()
    kp = O.lowered_k(k, ns)
    vp = empty((o, kp // 2), np.uint16)
    mp = empty((o, (kp + 7) // 8), np.uint8)
    S.nm_lower_slide(v, i, o, k, ns, vp, mp, S.NM_META_2BIT)
    y = empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(S.NM_W_SLIDE, t, o, k, dev(x), vp, y, ns=ns, w_meta=mp, w_meta_fmt=S.NM_META_2BIT)
    S.nm_spmm(a)
    sync()
    pruned, _ = O.sparsify(w, 2 * ns - 2, 2 * ns)
    check_gemm(host(y, np.float32), O.gemm(x, pruned), x, pruned, label=f"slide ns={ns}")


def test_spmm_w_slide_full_size_sampled():
    """6:8 weights 4096x4096 lowered to 2:4 over K'=6144, T in {1,16,128,4096}: every output
    written, whole-output projections, the oracle on one row of every 128-row band."""
    d = synth.slide_6of8_layer(t_max=4096)
    x_all, w = d["x"], d["w"]
    o, k = w.shape
    vp, mp = slide_pack_gpu(w, 4)
    sync()
    pruned, _ = O.sparsify(w, 6, 8)
    rows_w = sample_rows(o, 32, seed=3)
    v, i = O.compress(w[rows_w], 6, 8)
    vp_ref, ip_ref = O.slide_lower(v, i, k, 4)
    assert (host(vp, np.uint16)[rows_w] == vp_ref).all()
    assert (host(mp, np.uint8)[rows_w] == O.pack_meta_2bit(ip_ref)).all()
    # with the workspace the size query asks for (the measured configuration: X lifted once,
    # positions K-blocked, direct-to-LDS product at 4096 tokens), and without one
    for t, ws in ((1, True), (16, True), (128, True), (4096, True), (4096, False)):
        x = x_all[:t]
        y = empty((t, o), np.float32, fill=float("nan"))
        a = mk_args(S.NM_W_SLIDE, t, o, k, dev(x), vp, y, ns=4, w_meta=mp, w_meta_fmt=S.NM_META_2BIT)
        if ws:
            nb = S.nm_spmm_workspace_size(a)
            wsb = empty((max(nb, 16),), np.uint8)
            a.workspace, a.workspace_bytes = wsb.data_ptr(), nb
        S.nm_spmm(a)
        sync()
        yh = host(y, np.float32)
        assert np.isfinite(yh).all(), f"slide full t={t}: unwritten outputs"
        check_projection(yh, O.bf16_to_f64(x), O.bf16_to_f64(pruned), label=f"slide full t={t} projection")
        rows = band_rows(t, 128, seed=t)
        check_gemm(yh[rows], O.gemm(x[rows], pruned), x[rows], pruned, label=f"slide full t={t} ws={ws}")


SPARSE_KERNELS = {"lds": ("tile_lds",), "lds_rowmeta": ("tile_lds", "no_meta_block"), "regs": ("tile_regs",),
                  "tile": ("few_tile",), "stream": ("few_stream",)}


@pytest.mark.parametrize("kernel,t,o", [("lds", 300, 264), ("lds", 130, 520),
                                        ("lds_rowmeta", 300, 264), ("regs", 300, 264),
                                        ("regs", 130, 520), ("tile", 33, 264), ("tile", 64, 520),
                                        ("tile", 100, 264), ("tile", 128, 130), ("stream", 100, 264)])
def test_sparse_weight_product_kernels(kernel, t, o):
    """2:4-weight products on each kernel: large-token direct-to-LDS and register-staged
    tiles, the few-token split-K tile kernel and the few-token streaming kernel.  Plain
    2:4, lowered 6:8 / 4:6 / 8:10 (X lifted into the workspace first where the kernel
    needs it) and the hybrid format with its dense second phase; ragged T and O."""
    print(f"sparse kernels kernel={kernel} t={t} o={o}", flush=True)
    rng = np.random.default_rng(t + o)
    with use_route(*SPARSE_KERNELS[kernel]):
        k = 1024
        x = synth.normal_bf16(rng, (t, k))
        w = synth.normal_bf16(rng, (o, k), 0.02)
        v, mt = gpu_compress_2of4(w)
        ws24, _ = O.sparsify(w, 2, 4)
        for ws in (True, False):
            y = run_w(S.NM_W_COMPRESSED, x, v, mt, o, k, workspace=ws)
            check_gemm(y, O.gemm(x, ws24), x, ws24, label=f"2:4 {kernel}")
        for ns, kk in ((4, 2048), (3, 1536), (5, 2560)):
            xs = synth.normal_bf16(rng, (t, kk))
            wsl = synth.normal_bf16(rng, (o, kk), 0.02)
            vv, ii = O.compress(wsl, 2 * ns - 2, 2 * ns)
            kp = O.lowered_k(kk, ns)
            vp = empty((o, kp // 2), np.uint16)
            mp = empty((o, (kp + 7) // 8), np.uint8)
            S.nm_lower_slide(dev(vv), dev(ii), o, kk, ns, vp, mp, S.NM_META_2BIT)
            pr, _ = O.sparsify(wsl, 2 * ns - 2, 2 * ns)
            for ws in (True, False):
                y = run_w(S.NM_W_SLIDE, xs, vp, mp, o, kk, ns=ns, workspace=ws)
                check_gemm(y, O.gemm(xs, pr), xs, pr, label=f"slide ns={ns} ws={ws} {kernel}")
        kd = 256
        sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
        sync()
        sp, de, hv, hi, hwd = O.hybrid_pack(w, kd)
        wh = w.copy()
        wh[:, sp] = O.decompress(hv, hi, 2, 4, k - kd)
        yh = run_hybrid(x, sc, k - kd, dc, kd, wv, wm, wdd, o)
        check_gemm(yh, O.hybrid_gemm(x, sp, de, hv, hi, hwd), x, wh, label=f"hybrid {kernel}")


# ----------------------------------------------------------------------- hybrid ---

def hybrid_pack_gpu(w, kd, fmt=S.NM_META_2BIT):
    o, k = w.shape
    ks = k - kd
    sc = empty((max(ks, 1),), np.int32, fill=-1)
    dc = empty((max(kd, 1),), np.int32, fill=-1)
    wv = empty((o, max(ks // 2, 1)), np.uint16, fill=-1)
    wm = empty((o, max((ks + 7) // 8 if fmt else ks // 2, 1)), np.uint8, fill=255)
    wdd = empty((o, max(kd, 8)), np.uint16, fill=-1)
    ws = empty((S.nm_hybrid_pack_workspace_size(k),), np.uint8)
    S.nm_hybrid_pack(dev(w), kd, sc, dc, wv, wm, fmt, wdd, ws, ldwd=max(kd, 8))
    return sc, dc, wv, wm, wdd


def run_hybrid(x, sc, ks, dc, kd, wv, wm, wdd, o, ldwd=None, accumulate=0):
    import ctypes
    t = x.shape[0]
    y = empty((t, o), np.float32, fill=float("nan"))
    route = _ROUTE["route"]
    nb = S.nm_hybrid_gemm_workspace_size(t, ks, kd, o, sc is not None or dc is not None, route)
    ws = empty((max(nb, 16),), np.uint8)
    rep = ctypes.c_uint32(0)
    S.nm_hybrid_gemm(dev(x), sc, ks, dc, kd, wv, wm, S.NM_META_2BIT, wdd, o, y, accumulate, ldwd=ldwd,
                     workspace=ws, workspace_bytes=nb, route=route, taken=rep)
    LAST_TAKEN[0] = rep.value
    sync()
    return host(y, np.float32)


@pytest.mark.parametrize("kind", ["act", "act_fp8", "w24", "slide", "slide_copy", "hybrid", "w8a8"])
@pytest.mark.parametrize("t", [200, 700])
def test_mid_range_split_tile(kind, t):
    """Above 128 tokens, shapes whose 256 x 256 output tiles would not fill the chip run on
    the split-K 128-row tile kernel with partial tiles in the workspace, for every weight
    kind on its default route: 8:16 activations (select, then the product) on bf16 and fp8
    weights, 2:4, lowered 6:8 with the lift in the tile loads or (lift_copy hint) staged,
    the hybrid format, fp8 weights with fp8 activations.  Ragged T and O (9 row tiles, 2 or
    6 token tiles), the oracle on every row; the no_few hint keeps the large-tile kernels."""
    print(f"mid-range split kind={kind} t={t}", flush=True)
    rng = np.random.default_rng(t + len(kind))
    o, k = 1040, 2048
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)

    def routes(fn, extra=()):
        with use_route(*extra):
            y = fn()
            tk = taken()
            assert {"tile_split", "tile_lds"} <= tk, (kind, tk)
            with use_route("no_few"):
                y_large = fn()
                assert "tile_split" not in taken(), (kind, taken())
        return y, y_large, tk

    if kind in ("act", "act_fp8"):
        sx, keep = O.sparsify(x, 8, 16)
        if kind == "act":
            ref, wv = O.gemm(sx, w), w
            fn = lambda: run_act(x, w, 8, 16)
        else:
            q, sc = synth.fp8_e4m3_quantize_rows(w)
            ref, wv = O.spmm_act_fp8(x, q, sc, 8, 16), O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
            fn = lambda: run_act(x, None, 8, 16, w8=q, s8=sc)
        (y, mask), (y_large, mask_large), tk = routes(fn)
        assert "select" in tk, tk
        assert (mask == O.pack_mask(keep)).all() and (mask_large == mask).all()
        for yy, lab in ((y, "split"), (y_large, "large")):
            check_gemm(yy, ref, sx, wv, label=f"mid {kind} t={t} {lab}")
    elif kind == "w24":
        v, mt = gpu_compress_2of4(w)
        pr, _ = O.sparsify(w, 2, 4)
        y, y_large, tk = routes(lambda: run_w(S.NM_W_COMPRESSED, x, v, mt, o, k))
        assert "sparse_mma" in tk, tk
        for yy, lab in ((y, "split"), (y_large, "large")):
            check_gemm(yy, O.gemm(x, pr), x, pr, label=f"mid 2:4 t={t} {lab}")
    elif kind in ("slide", "slide_copy"):
        vp, mp = slide_pack_gpu(w, 4)
        pr, _ = O.sparsify(w, 6, 8)
        extra = ("lift_copy",) if kind == "slide_copy" else ()
        y, y_large, tk = routes(lambda: run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=4), extra)
        assert ("lift" in tk) == (kind == "slide_copy"), tk
        for yy, lab in ((y, "split"), (y_large, "large")):
            check_gemm(yy, O.gemm(x, pr), x, pr, label=f"mid {kind} t={t} {lab}")
    elif kind == "hybrid":
        kd = 256
        sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
        sync()
        sp, de, hv, hi, hwd = O.hybrid_pack(w, kd)
        wh = w.copy()
        wh[:, sp] = O.decompress(hv, hi, 2, 4, k - kd)
        y, y_large, tk = routes(lambda: run_hybrid(x, sc, k - kd, dc, kd, wv, wm, wdd, o))
        ref = O.hybrid_gemm(x, sp, de, hv, hi, hwd)
        for yy, lab in ((y, "split"), (y_large, "large")):
            check_gemm(yy, ref, x, wh, label=f"mid hybrid t={t} {lab}")
    else:
        w8, idx, wsc = w8a8_weights(rng, o, k, 4)
        ref = O.spmm_w8a8_slide(x, w8, idx, wsc, k, 4)
        a_v, b_v = w8a8_operands(x, w8, idx, wsc, k, 4)
        y, y_large, tk = routes(lambda: run_w8a8(x, w8, idx, wsc, o, k, 4))
        assert "quant" in tk, tk
        for yy, lab in ((y, "split"), (y_large, "large")):
            check_gemm_vals(yy, ref, a_v, b_v, label=f"mid w8a8 t={t} {lab}")


# shapes whose 256 x 256 tiles fill under one round with long reductions: (t, o, k) with
# ragged T and O; 90 tiles split in two, 72 tiles split in three
LARGE_SPLIT = {"act": (2500, 2056, 12800), "act_fp8": (2500, 2056, 12800), "act_pts": (2500, 2056, 12800),
               "w24": (1800, 2056, 6144), "slide": (1800, 2056, 8192), "hybrid": (1800, 2056, 6144),
               "w8a8": (2500, 2056, 8192)}


@pytest.mark.parametrize("kind", list(LARGE_SPLIT))
def test_large_tile_split(kind):
    """Above 128 tokens, 256 x 256 tiles that fill under one round of workgroups, with
    enough K-steps per range, have their reduction split in two to four ranges (partial
    tiles in the workspace, summed in range order): 8:16 activations on bf16 and fp8
    weights and with the mitigations' epilogue (D-PTS + VAR), 2:4, lowered 6:8 with the
    lift in the loads, the hybrid format and fp8 x fp8, the sparse ones on K-blocked
    positions.  Every output written; the oracle on one row of every 256-row band and the
    last row."""
    t, o, k = LARGE_SPLIT[kind]
    print(f"large tile split kind={kind} t={t} o={o} k={k}", flush=True)
    rng = np.random.default_rng(t + o + len(kind))
    rows = np.unique(np.r_[np.minimum(np.arange(0, t, 256) + rng.integers(0, 256, (t + 255) // 256), t - 1), t - 1])
    x = (pts_rows(rng, t, k) if kind == "act_pts" else synth.student_t_bf16(rng, (t, k), 4.0, 0.5))
    w = synth.normal_bf16(rng, (o, k), 0.02)
    if kind in ("act", "act_fp8"):
        sx, keep = O.sparsify(x[rows], 8, 16)
        if kind == "act":
            y, _ = run_act(x, w, 8, 16, want_mask=False)
            ref, wv = O.gemm(sx, w), w
        else:
            q, sc = synth.fp8_e4m3_quantize_rows(w)
            y, _ = run_act(x, None, 8, 16, w8=q, s8=sc, want_mask=False)
            ref, wv = O.spmm_act_fp8(x[rows], q, sc, 8, 16), O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
        tk = taken()
        assert np.isfinite(y).all(), kind
        check_gemm(y[rows], ref, sx, wv, label=f"large split {kind}")
    elif kind == "act_pts":
        pts = S.NM_PTS_DYNAMIC | S.NM_PTS_VAR
        y, mask = run_spmm_pts(x, w, 8, 16, pts)
        tk = taken()
        ref, sp_, keep, alpha, beta, v = pts_reference(x[rows], w, O.bf16_to_f64(w), 8, 16, pts, None)
        assert (mask[rows] == O.pack_mask(keep)).all()
        assert np.isfinite(y).all(), kind
        check_pts(y[rows], ref, sp_, O.bf16_to_f64(w), alpha, beta, v, label="large split pts")
    elif kind == "w24":
        v, mt = gpu_compress_2of4(w)
        pr, _ = O.sparsify(w, 2, 4)
        y = run_w(S.NM_W_COMPRESSED, x, v, mt, o, k)
        tk = taken()
        assert np.isfinite(y).all(), kind
        check_gemm(y[rows], O.gemm(x[rows], pr), x[rows], pr, label="large split 2:4")
    elif kind == "slide":
        vp, mp = slide_pack_gpu(w, 4)
        pr, _ = O.sparsify(w, 6, 8)
        y = run_w(S.NM_W_SLIDE, x, vp, mp, o, k, ns=4)
        tk = taken()
        assert "lift" not in tk, tk
        assert np.isfinite(y).all(), kind
        check_gemm(y[rows], O.gemm(x[rows], pr), x[rows], pr, label="large split 6:8")
    elif kind == "hybrid":
        kd = 1024
        sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
        sync()
        sp, de, hv, hi, hwd = O.hybrid_pack(w, kd)
        wh = w.copy()
        wh[:, sp] = O.decompress(hv, hi, 2, 4, k - kd)
        y = run_hybrid(x, sc, k - kd, dc, kd, wv, wm, wdd, o)
        tk = taken()
        assert np.isfinite(y).all(), kind
        check_gemm(y[rows], O.hybrid_gemm(x[rows], sp, de, hv, hi, hwd), x[rows], wh, label="large split hybrid")
    else:
        w8, idx, wsc = w8a8_weights(rng, o, k, 4)
        y = run_w8a8(x, w8, idx, wsc, o, k, 4)
        tk = taken()
        assert "quant" in tk, tk
        assert np.isfinite(y).all(), kind
        a_v, b_v = w8a8_operands(x[rows], w8, idx, wsc, k, 4)
        check_gemm_vals(y[rows], O.spmm_w8a8_slide(x[rows], w8, idx, wsc, k, 4), a_v, b_v, label="large split w8a8")
    assert {"tile_split", "tile_lds", "reduce"} <= tk, (kind, tk)
    if kind in ("w24", "slide", "hybrid", "w8a8"):
        assert {"meta_block", "sparse_mma"} <= tk, (kind, tk)


@pytest.mark.parametrize("kind", ["act", "act_fp8"])
def test_large_half_tiles(kind):
    """Dense-weight products whose 256 x 256 tiles would have their reduction split (99
    tiles, 200 K-steps) while 256 x 128 tiles fill three quarters to one round (198) take
    the unsplit half tiles: no partial tiles, no second pass.  8:16 activations on bf16
    and fp8 weights; every output written, the oracle on one row of every 256-row band and
    the last row."""
    t, o, k = 2800, 2056, 12800
    print(f"large half tiles kind={kind} t={t} o={o} k={k}", flush=True)
    rng = np.random.default_rng(t + o + len(kind))
    rows = np.unique(np.r_[np.minimum(np.arange(0, t, 256) + rng.integers(0, 256, (t + 255) // 256), t - 1), t - 1])
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    sx, keep = O.sparsify(x[rows], 8, 16)
    if kind == "act":
        y, _ = run_act(x, w, 8, 16, want_mask=False)
        ref, wv = O.gemm(sx, w), w
    else:
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        y, _ = run_act(x, None, 8, 16, w8=q, s8=sc, want_mask=False)
        ref, wv = O.spmm_act_fp8(x[rows], q, sc, 8, 16), O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    tk = taken()
    assert "tile_lds" in tk and "tile_split" not in tk and "reduce" not in tk, (kind, tk)
    assert np.isfinite(y).all(), kind
    check_gemm(y[rows], ref, sx, wv, label=f"large half tiles {kind}")


@pytest.mark.parametrize("t,o,kc", [(300, 264, 1088), (257, 130, 64), (512, 520, 2112)])
def test_blocked_positions_match_row_major(t, o, kc):
    """The large-token 2:4 product reads the weight positions from a K-blocked copy in the
    workspace; under the no_meta_block hint it reads them row-major.  Only the source of the same
    bytes differs, so the two outputs agree bit for bit; both match the oracle.  Ragged
    step counts (17, 1, 33 K-steps of 64) and row counts; plain 2:4 and the hybrid format."""
    print(f"blocked positions t={t} o={o} kc={kc}", flush=True)
    rng = np.random.default_rng(t + o + kc)
    x = synth.normal_bf16(rng, (t, kc))
    w = synth.normal_bf16(rng, (o, kc), 0.02)
    v, mt = gpu_compress_2of4(w)
    ws24, _ = O.sparsify(w, 2, 4)
    with use_route("tile_lds"):
        y_blk = run_w(S.NM_W_COMPRESSED, x, v, mt, o, kc)
        assert "meta_block" in taken()
        with use_route("no_meta_block"):
            y_row = run_w(S.NM_W_COMPRESSED, x, v, mt, o, kc)
            assert "meta_block" not in taken() and "tile_lds" in taken()
    assert np.array_equal(y_blk.view(np.uint32), y_row.view(np.uint32)), "blocked vs row-major positions"
    check_gemm(y_blk, O.gemm(x, ws24), x, ws24, label="2:4 blocked positions")
    kd = 64
    xh = synth.normal_bf16(rng, (t, kc + kd))
    wh0 = synth.normal_bf16(rng, (o, kc + kd), 0.02)
    sc, dc, wv, wm, wdd = hybrid_pack_gpu(wh0, kd)
    sync()
    sp, de, hv, hi, hwd = O.hybrid_pack(wh0, kd)
    wh = wh0.copy()
    wh[:, sp] = O.decompress(hv, hi, 2, 4, kc)
    with use_route("tile_lds"):
        yh_blk = run_hybrid(xh, sc, kc, dc, kd, wv, wm, wdd, o)
        assert "meta_block" in taken()
        with use_route("no_meta_block"):
            yh_row = run_hybrid(xh, sc, kc, dc, kd, wv, wm, wdd, o)
            assert "meta_block" not in taken()
    assert np.array_equal(yh_blk.view(np.uint32), yh_row.view(np.uint32)), "hybrid blocked vs row-major"
    check_gemm(yh_blk, O.hybrid_gemm(xh, sp, de, hv, hi, hwd), xh, wh, label="hybrid blocked positions")


@pytest.mark.parametrize("o,k,kd", [(100, 256, 64), (64, 128, 0), (48, 96, 96), (300, 512, 128)])
def test_hybrid_pack_and_gemm(o, k, kd):
    rng = np.random.default_rng(o + k + kd)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    x = synth.normal_bf16(rng, (130, k))
    sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
    sync()
    sp, de, v, i, wd = O.hybrid_pack(w, kd)
    ks = k - kd
    if ks:
        assert (host(sc, np.int32)[:ks] == sp).all()
        assert (host(wv, np.uint16)[:, :ks // 2] == v).all()
        assert (host(wm, np.uint8)[:, :(ks + 7) // 8] == O.pack_meta_2bit(i)).all()
    if kd:
        assert (host(dc, np.int32)[:kd] == de).all()
        assert (host(wdd, np.uint16)[:, :kd] == wd).all()
    wh = w.copy()
    if ks:
        wh[:, sp] = O.decompress(v, i, 2, 4, ks)
    for t in (130, 5, 40):
        xt = np.ascontiguousarray(x[:t])
        y = run_hybrid(xt, sc if ks else None, ks, dc if kd else None, kd, wv, wm, wdd if kd else None, o,
                       ldwd=max(kd, 8))
        check_gemm(y, O.hybrid_gemm(xt, sp, de, v, i, wd), xt, wh, label=f"hybrid t={t}")


def test_hybrid_prepermuted_input():
    """Column lists NULL: x already holds the sparse region then the dense region."""
    rng = np.random.default_rng(21)
    o, k, kd = 136, 512, 128
    w = synth.normal_bf16(rng, (o, k), 0.02)
    x = synth.normal_bf16(rng, (70, k))
    sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
    sync()
    sp, de, v, i, wd = O.hybrid_pack(w, kd)
    xp = np.ascontiguousarray(np.concatenate([x[:, sp], x[:, de]], axis=1))
    wh = w.copy()
    wh[:, sp] = O.decompress(v, i, 2, 4, k - kd)
    for t in (70, 3):
        y = run_hybrid(np.ascontiguousarray(xp[:t]), None, k - kd, None, kd, wv, wm, wdd, o, ldwd=max(kd, 8))
        check_gemm(y, O.hybrid_gemm(x[:t], sp, de, v, i, wd), x[:t], wh, label=f"hybrid prepermuted t={t}")
    # the gathered form needs its staging workspace
    y = empty((3, o), np.float32)
    st = S.nm_hybrid_gemm(dev(x[:3]), sc, k - kd, dc, kd, wv, wm, S.NM_META_2BIT, wdd, o, y, ldwd=max(kd, 8),
                          check=False)
    assert st == S.NM_EINVAL


def test_hybrid_full_size_sampled():
    """W 14336x4096, 25% dense columns; T in {1, 8, 32, 64, 2048}: every output written,
    whole-output projections, the oracle on one row of every 128-row band."""
    d = synth.hybrid_up_layer(t_max=2048)
    x_all, w, kd = d["x"], d["w"], d["k_dense"]
    o, k = w.shape
    sc, dc, wv, wm, wdd = hybrid_pack_gpu(w, kd)
    sync()
    sp, de = O.hybrid_columns(w, kd)
    assert (host(sc, np.int32) == sp).all() and (host(dc, np.int32) == de).all()
    rows_w = sample_rows(o, 64, seed=4)
    ws_ref = O.sparsify(np.ascontiguousarray(w[rows_w][:, sp]), 2, 4)[0]
    v, i = O.compress(np.ascontiguousarray(w[rows_w][:, sp]), 2, 4)
    assert (host(wv, np.uint16)[rows_w] == v).all()
    assert (host(wm, np.uint8)[rows_w] == O.pack_meta_2bit(i)).all()
    assert (host(wdd, np.uint16)[rows_w] == w[rows_w][:, de]).all()
    wh = w.copy()
    wh[:, sp] = O.sparsify(np.ascontiguousarray(w[:, sp]), 2, 4)[0]
    del ws_ref
    hv_full, hi_full = O.compress(np.ascontiguousarray(w[:, sp]), 2, 4)
    hwd_full = np.ascontiguousarray(w[:, de])
    for t in (1, 8, 32, 64, 2048):
        x = x_all[:t]
        y = run_hybrid(x, sc, k - kd, dc, kd, wv, wm, wdd, o)
        assert np.isfinite(y).all(), f"hybrid full t={t}: unwritten outputs"
        check_projection(y, O.bf16_to_f64(x), O.bf16_to_f64(wh), label=f"hybrid full t={t} projection")
        rows = band_rows(t, 128, seed=t)
        check_gemm(y[rows], O.hybrid_gemm(x[rows], sp, de, hv_full, hi_full, hwd_full), x[rows], wh,
                   label=f"hybrid full t={t}")


# --------------------------------------------------------- fp8 x fp8 (W8A8) ---

@pytest.mark.parametrize("ns,t,k,pad", [(4, 37, 1024, 0), (2, 5, 256, 16), (3, 64, 96, 32), (4, 1, 64, 48),
                                      (4, 3, 2056, 0), (4, 2, 8192, 16), (4, 2, 8200, 0)])
def test_quant_lift_bitexact(ns, t, k, pad):
    """Per-token e4m3 codes (lifted) and scales bit for bit against the oracle: Student-t
    rows, an all-zero row, tiny values (subnormal codes), ties of the largest magnitude."""
    print(f"quant lift ns={ns} t={t} k={k} pad={pad}", flush=True)
    import torch

    rng = np.random.default_rng(ns * 100 + t + k)
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    if t > 3:
        x[1] = 0
        x[2] = rng.choice(np.array([0x0001, 0x8002, 0x0100, 0x3F80, 0xBF80], np.uint16), size=k)
        x[3, : k // 2] = x[3, 0]
    kp = O.lowered_k(k, ns) if ns > 2 else k
    ldq = (kp + 15) // 16 * 16 + pad
    xq = torch.full((t, ldq), 0x55, dtype=torch.uint8, device="cuda")
    xs = torch.empty((t,), dtype=torch.float32, device="cuda")
    S.nm_quant_lift(dev(x), ns, xq, xs)
    sync()
    q, s_ref = O.quantize_tokens(x)
    q_ref = O.lift(q, ns).astype(np.uint8) if ns > 2 else q
    got = xq.cpu().numpy()
    assert (got[:, :kp] == q_ref).all()
    assert (got[:, kp:] == 0).all()
    assert (xs.cpu().numpy().view(np.uint32) == s_ref.view(np.uint32)).all()


def w8a8_weights(rng, o, k, ns):
    """fp8 weights of the lowered 2:4 form: a random bf16 W pruned (2N-2):2N (2:4 for
    N = 2), lowered by the oracle, the kept values quantized per row (input format)."""
    w = synth.normal_bf16(rng, (o, k), 0.02)
    if ns == 2:
        vals, idx = O.compress(w, 2, 4)
    else:
        v, i = O.compress(w, 2 * ns - 2, 2 * ns)
        vals, idx = O.slide_lower(v, i, k, ns)
    w8, ws = synth.fp8_e4m3_quantize_rows(vals)
    return w8, idx, ws


def run_w8a8(x, w8, idx, ws, o, k, ns, accumulate=0, y0=None, rows=None):
    import torch

    t = x.shape[0]
    mode = S.NM_W_SLIDE if ns > 2 else S.NM_W_COMPRESSED
    y = dev(y0.astype(np.float32)) if y0 is not None else empty((t, o), np.float32, fill=float("nan"))
    a = mk_args(mode, t, o, k, dev(x), dev(w8), y, ns=ns, w_dtype=S.NM_W_FP8E4M3, w_scale=dev(ws),
                         w_meta=dev(O.pack_meta_2bit(idx)), w_meta_fmt=S.NM_META_2BIT, accumulate=accumulate)
    nb = S.nm_spmm_workspace_size(a)
    wsb = empty((max(nb, 16),), np.uint8)
    a.workspace, a.workspace_bytes = wsb.data_ptr(), nb
    spmm_call(a)
    sync()
    if rows is None:
        return host(y, np.float32)
    return y[torch.from_numpy(rows).cuda()].cpu().numpy()


def w8a8_operands(x, w8, idx, ws, k, ns):
    q, s_t = O.quantize_tokens(x)
    qx = O.lift(q, ns).astype(np.uint8) if ns > 2 else q
    kp = qx.shape[1]
    wd = O.decompress(w8.astype(np.uint16), idx, 2, 4, kp).astype(np.uint8)
    return (O.fp8_e4m3_to_f64(qx) * s_t[:, None].astype(np.float64),
            O.fp8_e4m3_to_f64(wd) * ws[:, None].astype(np.float64))


@pytest.mark.parametrize("ns", [2, 4])
@pytest.mark.parametrize("t,o", [(1, 264), (17, 520), (64, 264), (128, 130), (200, 264), (600, 520)])
def test_spmm_w8a8(ns, t, o):
    """fp8 weights and per-token fp8 activations on the fp8 sparse matrix instruction:
    plain 2:4 and 6:8 lowered (activations lifted in the quantizing pass), every token
    route (split reduction for few tokens, 256 x 256 tiles above), ragged O, accumulate."""
    print(f"w8a8 ns={ns} t={t} o={o}", flush=True)
    rng = np.random.default_rng(ns * 1000 + t + o)
    k = 1024
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w8, idx, ws = w8a8_weights(rng, o, k, ns)
    ref = O.spmm_w8a8_slide(x, w8, idx, ws, k, ns)
    a_v, b_v = w8a8_operands(x, w8, idx, ws, k, ns)
    y = run_w8a8(x, w8, idx, ws, o, k, ns)
    check_gemm_vals(y, ref, a_v, b_v, label=f"w8a8 ns={ns}")
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    y2 = run_w8a8(x, w8, idx, ws, o, k, ns, accumulate=1, y0=y0)
    check_gemm_vals(y2.astype(np.float64) - y0, ref, a_v, b_v, label=f"w8a8 ns={ns} accumulate")


@pytest.mark.parametrize("ns", [2, 4])
@pytest.mark.parametrize("t,o", [(1, 264), (1, 100), (3, 264), (16, 520)])
def test_spmm_w8a8_stream(ns, t, o):
    """fp8 weights and per-token fp8 activations at up to 16 tokens: the quantizing pass,
    then the weight-streaming kernel on the e4m3 2:4 codes (widened to bf16 after their
    LDS read, the one-token X row staged in LDS), against the oracle and against the
    split tile kernel on the fp8 instruction (the NM_ROUTE_FEW_TILE hint).  The reduction
    (K' = 1152 or 1920) leaves half a stage for the register path."""
    print(f"w8a8 stream ns={ns} t={t} o={o}", flush=True)
    rng = np.random.default_rng(ns * 100 + t + o)
    k = 1152 if ns == 2 else 1280
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w8, idx, ws = w8a8_weights(rng, o, k, ns)
    ref = O.spmm_w8a8_slide(x, w8, idx, ws, k, ns)
    a_v, b_v = w8a8_operands(x, w8, idx, ws, k, ns)
    y = run_w8a8(x, w8, idx, ws, o, k, ns)
    tk = taken()
    assert {"quant", "few_stream", "sparse_mma"} <= tk and "tile_split" not in tk, tk
    if t == 1:
        assert "few_xlds" in tk, tk
    check_gemm_vals(y, ref, a_v, b_v, label=f"w8a8 stream ns={ns} t={t}")
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    y2 = run_w8a8(x, w8, idx, ws, o, k, ns, accumulate=1, y0=y0)
    check_gemm_vals(y2.astype(np.float64) - y0, ref, a_v, b_v, label=f"w8a8 stream ns={ns} t={t} accumulate")
    with use_route("few_tile"):
        yt = run_w8a8(x, w8, idx, ws, o, k, ns)
        assert "few_stream" not in taken(), taken()
    check_gemm_vals(yt, ref, a_v, b_v, label=f"w8a8 tile ns={ns} t={t}")
    if t == 1:
        # the separate quantizing pass with X fragments in registers (the one-token kernel
        # otherwise quantizes the row in LDS itself): the same codes and scale, so the same
        # products, summed in the same order
        with use_route("no_xlds"):
            yr = run_w8a8(x, w8, idx, ws, o, k, ns)
            assert "few_xlds" not in taken() and "quant" in taken(), taken()
        check_gemm_vals(yr, ref, a_v, b_v, label=f"w8a8 stream registers ns={ns}")


def test_spmm_w8a8_full_size_sampled():
    """6:8 weights 4096 x 4096 lowered to 2:4 over K' = 6144, fp8 weights and activations,
    T in {1, 128, 4096}: every output written, whole-output projections, the oracle on one
    row of every 128-row band."""
    print("w8a8 full", flush=True)
    d = synth.slide_6of8_layer(t_max=4096)
    x_all, w = d["x"], d["w"]
    o, k = w.shape
    v, i = O.compress(w, 6, 8)
    vals, idx = O.slide_lower(v, i, k, 4)
    w8, ws = synth.fp8_e4m3_quantize_rows(vals)
    for t in (1, 128, 4096):
        x = x_all[:t]
        y = run_w8a8(x, w8, idx, ws, o, k, 4)
        assert np.isfinite(y).all(), f"w8a8 full t={t}: unwritten outputs"
        a_all, b_v = w8a8_operands(x, w8, idx, ws, k, 4)
        check_projection(y, a_all, b_v, label=f"w8a8 full t={t} projection")
        rows = band_rows(t, 128, seed=t)
        ref = O.spmm_w8a8_slide(x[rows], w8, idx, ws, k, 4)
        check_gemm_vals(y[rows], ref, a_all[rows], b_v, label=f"w8a8 full t={t}")


# ------------------------------------------------------------------ Spense GLU ---

def spense_order_gpu(wg, wu, wd, hs_in, hs_mid, n_dense, strategy):
    import torch

    i_n, h = wg.shape
    perm = torch.empty((i_n,), dtype=torch.int32, device="cuda")
    scores = torch.empty((i_n,), dtype=torch.float64, device="cuda")
    ws = empty((max(S.nm_spense_glu_order_workspace_size(i_n), 16),), np.uint8)
    S.nm_spense_glu_order(dev(wg), dev(wu), dev(wd), torch.from_numpy(hs_in).cuda(),
                          torch.from_numpy(hs_mid).cuda(), n_dense, strategy, perm, ws, scores=scores)
    sync()
    return perm.cpu().numpy(), scores.cpu().numpy()


@pytest.mark.parametrize("i_n,h,n_dense", [(200, 64, 50), (40, 24, 0), (64, 8, 64), (136, 40, 33)])
def test_spense_glu_order(i_n, h, n_dense):
    """Loss-aware scores bit for bit (fp64, fixed order) and the permutation exactly, with
    forced score ties (repeated rows); the tail strategy gives the identity."""
    print(f"spense order i={i_n} h={h} dense={n_dense}", flush=True)
    rng = np.random.default_rng(i_n + h)
    wg = synth.normal_bf16(rng, (i_n, h), 0.02)
    wu = synth.normal_bf16(rng, (i_n, h), 0.02)
    wd = synth.normal_bf16(rng, (h, i_n), 0.02)
    wg[5], wu[5], wd[:, 5] = wg[3], wu[3], wd[:, 3]               # equal scores at 3 and 5
    hs_in = np.abs(rng.standard_normal(h)) + 0.1
    hs_mid = np.abs(rng.standard_normal(i_n)) + 0.1
    hs_mid[5] = hs_mid[3]
    perm, scores = spense_order_gpu(wg, wu, wd, hs_in, hs_mid, n_dense, S.NM_SPENSE_LOSS)
    ref = O.spense_glu_scores(wg, wu, wd, hs_in, hs_mid)
    assert scores[3] == scores[5]
    assert (scores.view(np.uint64) == ref.view(np.uint64)).all()
    assert (perm == O.spense_order(ref, n_dense)).all()
    perm_t, _ = spense_order_gpu(wg, wu, wd, hs_in, hs_mid, n_dense, S.NM_SPENSE_TAIL)
    assert (perm_t == O.spense_order_tail(i_n, n_dense)).all()


def test_spense_glu_order_full_size():
    """The 8B-shaped layer's MLP (gate/up 14336 x 4096, down 4096 x 14336), Hessian roots
    from the layer's input streams, 25% dense: scores bit for bit, permutation exactly."""
    print("spense order full", flush=True)
    lay = synth.transformer_layer(t_max=256, names=("gate", "up", "down"))
    wg, wu, wd = lay["w"]["gate"], lay["w"]["up"], lay["w"]["down"]
    hs_in = np.sqrt((O.bf16_to_f64(lay["x"]["mlp_in"]) ** 2).sum(0))
    hs_mid = np.sqrt((O.bf16_to_f64(lay["x"]["down_in"]) ** 2).sum(0))
    n_dense = wg.shape[0] // 4
    perm, scores = spense_order_gpu(wg, wu, wd, hs_in, hs_mid, n_dense, S.NM_SPENSE_LOSS)
    ref = O.spense_glu_scores(wg, wu, wd, hs_in, hs_mid)
    assert (scores.view(np.uint64) == ref.view(np.uint64)).all()
    assert (perm == O.spense_order(ref, n_dense)).all()


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("axis,o,k,ns", [(0, 100, 64, 60), (0, 48, 40, 0), (0, 40, 32, 40), (1, 24, 96, 64),
                                         (1, 130, 40, 0), (1, 20, 48, 48)])
def test_spense_pack(fmt, axis, o, k, ns):
    """Split by a random permutation: the 2:4 region's values and positions and the dense
    region bit for bit, rows (output-split) and columns (input-split)."""
    print(f"spense pack axis={axis} o={o} k={k} ns={ns} fmt={fmt}", flush=True)
    import torch

    rng = np.random.default_rng(o + k + ns + axis)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    n = o if axis == 0 else k
    perm = rng.permutation(n).astype(np.int32)
    v_ref, i_ref, wd_ref = O.spense_pack(w, perm, ns, axis)
    srows, kc = (ns, k) if axis == 0 else (o, ns)
    vals = empty((max(srows, 1), max(kc // 2, 1)), np.uint16, fill=-1)
    meta = empty((max(srows, 1), max((kc + 7) // 8 if fmt else kc // 2, 1)), np.uint8, fill=255)
    drows, dcols = wd_ref.shape
    ldwd = max((dcols + 7) // 8 * 8, 8)
    wdd = empty((max(drows, 1), ldwd), np.uint16, fill=-1)
    nb = S.nm_spense_pack_workspace_size(o, k, axis, ns)
    ws = empty((max(nb, 16),), np.uint8)
    S.nm_spense_pack(dev(w), axis, torch.from_numpy(perm).cuda(), ns, vals, meta, fmt, wdd, ws,
                     ldwd=ldwd, workspace_bytes=nb)
    sync()
    if srows and kc:
        assert (host(vals, np.uint16)[:srows, :kc // 2] == v_ref).all()
        got_meta = host(meta, np.uint8)[:srows]
        assert (got_meta[:, :(kc + 7) // 8] == O.pack_meta_2bit(i_ref)).all() if fmt else \
            (got_meta[:, :kc // 2] == i_ref).all()
    if drows and dcols:
        assert (host(wdd, np.uint16)[:drows, :dcols] == wd_ref).all()


@pytest.mark.parametrize("t", [1, 17, 64, 130, 600])
@pytest.mark.parametrize("o_s,o_d", [(264, 88), (0, 96), (128, 0), (2048, 512)])
def test_spense_outsplit_gemm(t, o_s, o_d):
    """Output-split product: y[:, :o_s] from the 2:4 rows, y[:, o_s:] from the dense rows,
    on every route (few tokens to large T), overwrite and accumulate."""
    print(f"spense outsplit t={t} o_s={o_s} o_d={o_d}", flush=True)
    import torch

    rng = np.random.default_rng(t + o_s + o_d)
    k = 1024
    o = o_s + o_d
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    perm = rng.permutation(o).astype(np.int32)
    v_ref, i_ref, wd_ref = O.spense_pack(w, perm, o_s, 0)
    ref = O.outsplit_gemm(x, v_ref, i_ref, wd_ref, k)
    w_eff = np.concatenate([O.decompress(v_ref, i_ref, 2, 4, k), wd_ref], 0) if o_s else wd_ref
    vals = empty((max(o_s, 1), k // 2), np.uint16)
    meta = empty((max(o_s, 1), k // 8), np.uint8)
    wdd = empty((max(o_d, 1), k), np.uint16)
    nb = S.nm_spense_pack_workspace_size(o, k, 0, o_s)
    ws = empty((max(nb, 16),), np.uint8)
    S.nm_spense_pack(dev(w), 0, torch.from_numpy(perm).cuda(), o_s, vals, meta, S.NM_META_2BIT, wdd, ws,
                     workspace_bytes=nb)
    y0 = rng.standard_normal((t, o)).astype(np.float32)
    for acc in (0, 1):
        y = dev(y0) if acc else empty((t, o), np.float32, fill=float("nan"))
        nb = S.nm_spense_outsplit_workspace_size(t, k, o_s, o_d)
        ws2 = empty((max(nb, 16),), np.uint8)
        S.nm_spense_outsplit_gemm(dev(x), vals, meta, o_s, wdd, o_d, y, acc, ws2, workspace_bytes=nb)
        sync()
        out = host(y, np.float32).astype(np.float64) - (y0 if acc else 0)
        check_gemm(out, ref, x, w_eff, label=f"outsplit acc={acc}")


def test_spense_down_input_split_prepermuted():
    """Down projection of the Spense MLP: columns packed by the permutation (input-split),
    product on an input that is already in the permuted order (no column lists)."""
    print("spense down", flush=True)
    import torch

    rng = np.random.default_rng(77)
    t, o, i_n, n_dense = 300, 520, 1024, 256
    w = synth.normal_bf16(rng, (o, i_n), 0.02)
    perm = rng.permutation(i_n).astype(np.int32)
    ns = i_n - n_dense
    v_ref, i_ref, wd_ref = O.spense_pack(w, perm, ns, 1)
    a = synth.student_t_bf16(rng, (t, i_n), 4.0, 0.5)             # GLU output, permuted order
    vals = empty((o, ns // 2), np.uint16)
    meta = empty((o, ns // 8), np.uint8)
    wdd = empty((o, n_dense), np.uint16)
    S.nm_spense_pack(dev(w), 1, torch.from_numpy(perm).cuda(), ns, vals, meta, S.NM_META_2BIT, wdd)
    sync()
    for tt in (1, 64, t):
        y = run_hybrid(a[:tt], None, ns, None, n_dense, vals, meta, wdd, o)
        ref = O.gemm(a[:tt, :ns], O.decompress(v_ref, i_ref, 2, 4, ns)) + O.gemm(a[:tt, ns:], wd_ref)
        w_eff = np.concatenate([O.decompress(v_ref, i_ref, 2, 4, ns), wd_ref], 1)
        check_gemm(y, ref, a[:tt], w_eff, label=f"spense down t={tt}")


# ------------------------------------------------------------------ edge cases ---

def test_zero_sizes_and_k_zero():
    y = empty((4, 8), np.float32, fill=5.0)
    x = empty((4, 8), np.uint16, fill=0)
    w = empty((8, 8), np.uint16, fill=0)
    a = mk_args(S.NM_ACT_DYNAMIC, 4, 8, 0, x, w, y, n=2, m=4, ldx=8, ldw=8)
    S.nm_spmm(a)
    sync()
    assert (host(y, np.float32) == 0).all()
    y.fill_(5.0)
    a.accumulate = 1
    S.nm_spmm(a)
    sync()
    assert (host(y, np.float32) == 5).all()
    a.t = 0
    assert S.nm_spmm(a, check=False) == S.NM_OK


def test_large_offsets_sampled():
    """Operands past 2^31 bytes: X 70000 x 16384 bf16 (2.3 GB, drawn on the GPU from a
    seeded generator), 8:16 activations into O = 256 through select, S(X) staged in a
    2.3 GB workspace and the direct-to-LDS product.  Mask and outputs on sampled rows,
    including rows whose byte offset is past 2^31 and the last row."""
    import torch
    print("large offsets t=70000 k=16384 o=256", flush=True)
    t, k, o = 70000, 16384, 256
    xd = synth.device_normal_bf16(torch, (t, k), seed=12)
    w = synth.normal_bf16(np.random.default_rng(13), (o, k), 0.02)
    y = empty((t, o), np.float32, fill=float("nan"))
    mask = empty((t, k // 32), np.uint32, fill=-1)
    a = mk_args(S.NM_ACT_DYNAMIC, t, o, k, xd, dev(w), y, n=8, m=16, x_mask_out=mask)
    nb = S.nm_spmm_workspace_size(a)
    assert nb >= t * k * 2
    ws = empty((nb,), np.uint8)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nb
    S.nm_spmm(a)
    sync()
    check_all_written(y, "large offsets")
    rows = np.array(sorted(set(band_rows(t, 4096, seed=3).tolist()) | {65535, 65536, 69999}))
    xr = xd[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
    sx, keep = O.sparsify(xr, 8, 16)
    assert (host(mask, np.uint32)[rows] == O.pack_mask(keep)).all()
    check_gemm(host(y, np.float32)[rows], O.gemm(sx, w), sx, w, label="large offsets")
    del ws, xd


# ------------------------------------------------------------ measurement probes ---

@pytest.mark.gpu
def test_measurement_probes():
    """The read probe XORs what each thread loads (one 16-byte element per thread when the
    buffer holds exactly one per thread); the matrix probe's sums scale with its round
    count (small integers, exact in fp32)."""
    print("probes", flush=True)
    import torch
    from semi_structured_sparse_amd import probe as P_
    nth = 2048 * 256
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2**32, size=(nth, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros((P_.nm_probe_sink_bytes() // 4,), dtype=torch.int32, device="cuda")
    P_.nm_probe_read(buf, nth * 16, sink)
    sync()
    got = sink[:nth].cpu().numpy().view(np.uint32)
    assert (got == (words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3])).all()
    outs = []
    for iters in (0, 3, 6):
        fs = torch.full((P_.nm_probe_sink_bytes() // 4,), float("nan"), dtype=torch.float32, device="cuda")
        P_.nm_probe_mfma(iters, fs)
        sync()
        outs.append(fs[:1024 * 256].cpu().numpy())
    assert (outs[0] == 0).all()
    assert np.isfinite(outs[1]).all() and (outs[1] > 0).all()
    assert (outs[2] == 2 * outs[1]).all()
    # contiguous blocks: block b XORs its run; with 4096 elements per block of 256 threads,
    # thread j of block b XORs elements b*4096 + j + 256*u, u < 16
    nel = 2048 * 4096
    w2 = rng.integers(0, 2**32, size=(nel, 4), dtype=np.uint64).astype(np.uint32)
    buf2 = torch.from_numpy(w2.view(np.int32)).cuda()
    sink2 = torch.zeros_like(sink)
    P_.nm_probe_read(buf2, nel * 16, sink2, mode=1)
    sync()
    x = np.bitwise_xor.reduce(w2.reshape(2048, 16, 256, 4), axis=1)          # [block][thread][4]
    ref = (x[..., 0] ^ x[..., 1] ^ x[..., 2] ^ x[..., 3]).reshape(-1)
    assert (sink2[:2048 * 256].cpu().numpy().view(np.uint32) == ref).all()
    # direct-to-LDS: 100 chunks of 16 KiB, one per wave; each lane reports the first dword
    # of its 16 bytes of the chunk's first KiB
    nch = 100
    P_.nm_probe_read(buf2, nch * 16384, sink2, mode=2)
    sync()
    got = sink2[:nch * 64].cpu().numpy().view(np.uint32).reshape(nch, 64)
    words = w2.reshape(-1)[:nch * 4096].reshape(nch, 16, 64, 4)                # chunk, KiB, lane, dword
    assert (got == words[:, 0, :, 0]).all()


@pytest.mark.parametrize("kind", ["act", "w24"])
@pytest.mark.parametrize("t,k", [(1, 14336), (1, 4096), (8, 4096)])
def test_few_token_half_rings(kind, t, k):
    """Past 256 row blocks (o = 8208: 513 blocks of 16 rows, the last ragged) the weight-
    streaming kernel runs 8 waves per workgroup on rings sized for 8, two workgroups per
    CU.  One token stages its X row beside the rings; a 14336-wide bf16 row does not fit
    twice per CU, so that call keeps whole rings and 16 waves (and the 2:4 one, whose whole
    rings leave no room for the row, reads X from global memory).  Forced 16 waves on whole
    rings partition the reduction differently: both against the oracle (8:16 activations
    with the mask, so the select pass runs apart; and 2:4 weights)."""
    print(f"few-token half rings kind={kind} t={t} k={k}", flush=True)
    o = 8208
    rng = np.random.default_rng(t * 31 + k)
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    if kind == "act":
        sx, keep = O.sparsify(x, 8, 16)
        ref, a_op, b_op = O.gemm(sx, w), sx, w
        run = lambda: run_act(x, w, 8, 16)
    else:
        ws24, _ = O.sparsify(w, 2, 4)
        v, mt = gpu_compress_2of4(w)
        ref, a_op, b_op = O.gemm(x, ws24), x, ws24
        run = lambda: (run_w(S.NM_W_COMPRESSED, x, v, mt, o, k), None)
    outs = {}
    for wpb in (0, 16):
        with use_route("few_stream", few_wpb=wpb):
            y, mask = run()
            assert "few_stream" in taken(), taken()
            if t == 1 and (kind == "act" or k == 4096):
                assert "few_xlds" in taken(), taken()
        if mask is not None:
            assert (mask == O.pack_mask(keep)).all()
        check_gemm(y, ref, a_op, b_op, label=f"{kind} t={t} k={k} wpb={wpb}")
        outs[wpb] = y
    assert not np.isnan(outs[0]).any()


def test_one_token_long_hybrid_row():
    """One token, hybrid input split over a 14336-wide row (10752 2:4 columns, then 3584
    dense, no column lists: the Spense down-projection form), 4096 outputs.  The staged
    row does not fit beside whole rings, so the call takes rings for 12 waves with the row
    in LDS; X read from global memory with 16 waves (no_xlds) partitions the reduction
    differently.  Both against the oracle."""
    print("one-token long hybrid row", flush=True)
    rng = np.random.default_rng(14336)
    o, ks, kd = 4096, 10752, 3584
    x = synth.normal_bf16(rng, (1, ks + kd))
    w = synth.normal_bf16(rng, (o, ks + kd), 0.02)
    wsp, _ = O.sparsify(np.ascontiguousarray(w[:, :ks]), 2, 4)
    vs, ms = gpu_compress_2of4(np.ascontiguousarray(w[:, :ks]))
    wd = np.ascontiguousarray(w[:, ks:])
    ref = O.gemm(np.ascontiguousarray(x[:, :ks]), wsp) + O.gemm(np.ascontiguousarray(x[:, ks:]), wd)
    wcat = np.concatenate([wsp, wd], axis=1)
    with use_route("few_stream"):
        y = run_hybrid(x, None, ks, None, kd, vs, ms, dev(wd), o)
        assert {"few_stream", "few_xlds"} <= taken(), taken()
        with use_route("no_xlds"):
            y_glb = run_hybrid(x, None, ks, None, kd, vs, ms, dev(wd), o)
            assert "few_xlds" not in taken(), taken()
    check_gemm(y, ref, x, wcat, label="hybrid row staged (12 waves)")
    check_gemm(y_glb, ref, x, wcat, label="hybrid row from global memory")


@pytest.mark.parametrize("o", [200, 4096])
def test_one_token_staged_x_bitexact(o):
    """One token on the weight-streaming kernel: X rows staged in LDS give the same bits as
    X read from global memory (the no_xlds hint), and match the oracle, for dense bf16 and
    fp8 weights (8:16 activations, ragged K), plain 2:4, lowered 6:8 and 4:6, and the
    two-segment hybrid; o = 200 also splits the reduction across workgroups."""
    print(f"one-token staged X o={o}", flush=True)
    rng = np.random.default_rng(o + 3)
    runs = []

    def both(label, fn):
        with use_route("few_stream"):
            y_lds = fn()
            assert {"few_stream", "few_xlds"} <= taken(), (label, taken())
            with use_route("no_xlds"):
                y_glb = fn()
                assert "few_stream" in taken() and "few_xlds" not in taken(), (label, taken())
        assert np.array_equal(y_lds.view(np.uint32), y_glb.view(np.uint32)), f"{label}: staged vs global X"
        runs.append(label)
        return y_lds

    k = 1056
    x = synth.student_t_bf16(rng, (1, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    sx, _ = O.sparsify(x, 8, 16)
    y = both("8:16 bf16", lambda: run_act(x, w, 8, 16)[0])
    check_gemm(y, O.gemm(sx, w), sx, w, label="8:16 bf16 staged")
    q, sc = synth.fp8_e4m3_quantize_rows(w)
    y = both("8:16 fp8", lambda: run_act(x, None, 8, 16, w8=q, s8=sc)[0])
    wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    check_gemm(y, O.spmm_act_fp8(x, q, sc, 8, 16), sx, wdeq, label="8:16 fp8 staged")
    v, mt = gpu_compress_2of4(w)
    ws24, _ = O.sparsify(w, 2, 4)
    y = both("w 2:4", lambda: run_w(S.NM_W_COMPRESSED, x, v, mt, o, k))
    check_gemm(y, O.gemm(x, ws24), x, ws24, label="w 2:4 staged")
    for ns in (4, 3):
        kk = 1008   # a multiple of 2 ns for both
        xs_ = np.ascontiguousarray(x[:, :kk])
        ws_ = np.ascontiguousarray(w[:, :kk])
        vp, mp = slide_pack_gpu(ws_, ns)
        pr, _ = O.sparsify(ws_, 2 * ns - 2, 2 * ns)
        y = both(f"slide ns={ns}", lambda: run_w(S.NM_W_SLIDE, xs_, vp, mp, o, kk, ns=ns))
        check_gemm(y, O.gemm(xs_, pr), xs_, pr, label=f"slide ns={ns} staged")
    kh, kd = 1024, 256
    xh = np.ascontiguousarray(x[:, :kh])
    wh0 = np.ascontiguousarray(w[:, :kh])
    sc_, dc_, wv, wm, wdd = hybrid_pack_gpu(wh0, kd)
    sync()
    sp, de, hv, hi, hwd = O.hybrid_pack(wh0, kd)
    whh = wh0.copy()
    whh[:, sp] = O.decompress(hv, hi, 2, 4, kh - kd)
    y = both("hybrid", lambda: run_hybrid(xh, sc_, kh - kd, dc_, kd, wv, wm, wdd, o, ldwd=kd))
    check_gemm(y, O.hybrid_gemm(xh, sp, de, hv, hi, hwd), xh, whh, label="hybrid staged")
    assert len(runs) == 6


@pytest.mark.parametrize("o", [200, 4096])
@pytest.mark.parametrize("m", [4, 8, 16, 32])
def test_one_token_select_in_kernel(m, o):
    """One token, n = m/2, no mask asked for: the weight-streaming kernel selects inside
    the X row it stages in LDS.  Same bits as the separate select pass followed by the
    product (the no_few_select hint), and within tolerance of the oracle, for bf16 and fp8
    weights; one row is Student-t, the other has many equal magnitudes (ties to the
    lower index)."""
    print(f"one-token select in kernel m={m} o={o}", flush=True)
    rng = np.random.default_rng(m * 100 + o)
    k = 1056 if m <= 16 else 1024
    w = synth.normal_bf16(rng, (o, k), 0.02)
    q, sc = synth.fp8_e4m3_quantize_rows(w)
    wdeq = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    xt = synth.student_t_bf16(rng, (1, k), 4.0, 0.5)
    # magnitudes from a few values and both signs: many ties inside each group
    vals = np.array([0x3F80, 0x4000, 0xBF80, 0xC000, 0x3F00, 0x0000, 0x8000], dtype=np.uint16)
    xtie = vals[rng.integers(0, len(vals), size=(1, k))].astype(np.uint16)
    for label, x in (("student-t", xt), ("ties", xtie)):
        sx, _ = O.sparsify(x, m // 2, m)
        with use_route("few_stream"):
            y_in = run_act(x, w, m // 2, m, want_mask=False)[0]
            assert {"few_select", "few_xlds"} <= taken() and "select" not in taken(), taken()
            y8_in = run_act(x, None, m // 2, m, w8=q, s8=sc, want_mask=False)[0]
            assert {"few_select", "few_xlds"} <= taken() and "select" not in taken(), taken()
            with use_route("no_few_select"):
                y_sep = run_act(x, w, m // 2, m, want_mask=False)[0]
                assert "select" in taken() and "few_select" not in taken(), taken()
                y8_sep = run_act(x, None, m // 2, m, w8=q, s8=sc, want_mask=False)[0]
                assert "select" in taken() and "few_select" not in taken(), taken()
        assert np.array_equal(y_in.view(np.uint32), y_sep.view(np.uint32)), f"{label} bf16: in-kernel vs separate"
        assert np.array_equal(y8_in.view(np.uint32), y8_sep.view(np.uint32)), f"{label} fp8: in-kernel vs separate"
        check_gemm(y_in, O.gemm(sx, w), sx, w, label=f"{label} {m // 2}:{m} bf16 in-kernel select")
        check_gemm(y8_in, O.spmm_act_fp8(x, q, sc, m // 2, m), sx, wdeq, label=f"{label} {m // 2}:{m} fp8")
    # accumulate into a nonzero y, both weight types
    y0 = rng.standard_normal((1, o)).astype(np.float32)
    with use_route("few_stream"):
        ya = run_act(xt, w, m // 2, m, accumulate=1, y0=y0, want_mask=False)[0]
        assert "few_select" in taken()
        ya8 = run_act(xt, None, m // 2, m, w8=q, s8=sc, accumulate=1, y0=y0, want_mask=False)[0]
        with use_route("no_few_select"):
            yb = run_act(xt, w, m // 2, m, accumulate=1, y0=y0, want_mask=False)[0]
            yb8 = run_act(xt, None, m // 2, m, w8=q, s8=sc, accumulate=1, y0=y0, want_mask=False)[0]
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), "accumulate bf16: in-kernel vs separate"
    assert np.array_equal(ya8.view(np.uint32), yb8.view(np.uint32)), "accumulate fp8: in-kernel vs separate"
    sxt, _ = O.sparsify(xt, m // 2, m)
    check_gemm(ya.astype(np.float64) - y0, O.gemm(sxt, w), sxt, w, label=f"{m // 2}:{m} in-kernel select accumulate")


def test_one_token_graph_replays():
    """One-token calls captured in a graph (X staged in LDS, selection inside the product;
    staged 2:4 weights; the hybrid with its permute): three replays, with eager calls and
    a synchronization between them, each bit-identical to the eager result."""
    print("one-token graph replays", flush=True)
    import torch
    rng = np.random.default_rng(77)
    o, k = 512, 1024
    x = synth.student_t_bf16(rng, (1, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    xd, wd_ = dev(x), dev(w)
    calls = []
    ya = empty((1, o), np.float32)
    stream = S.route_bits("few_stream")
    a = mk_args(S.NM_ACT_DYNAMIC, 1, o, k, xd, wd_, ya, n=8, m=16, route=stream)
    wsa = empty((max(S.nm_spmm_workspace_size(a), 16),), np.uint8)
    a.workspace, a.workspace_bytes = wsa.data_ptr(), S.nm_spmm_workspace_size(a)
    calls.append(("8:16 act", lambda: S.nm_spmm(a), ya))
    v, mt = gpu_compress_2of4(w)
    yw = empty((1, o), np.float32)
    b = mk_args(S.NM_W_COMPRESSED, 1, o, k, xd, v, yw, w_meta=mt, w_meta_fmt=S.NM_META_2BIT, route=stream)
    wsb = empty((max(S.nm_spmm_workspace_size(b), 16),), np.uint8)
    b.workspace, b.workspace_bytes = wsb.data_ptr(), S.nm_spmm_workspace_size(b)
    calls.append(("w 2:4", lambda: S.nm_spmm(b), yw))
    kd = 256
    sc_, dc_, wv, wm, wdd = hybrid_pack_gpu(w, kd)
    yh = empty((1, o), np.float32)
    nbh = S.nm_hybrid_gemm_workspace_size(1, k - kd, kd, o, True, stream)
    wsh = empty((max(nbh, 16),), np.uint8)
    import ctypes
    hrep = ctypes.c_uint32(0)
    calls.append(("hybrid", lambda: S.nm_hybrid_gemm(xd, sc_, k - kd, dc_, kd, wv, wm, S.NM_META_2BIT, wdd, o, yh,
                                                     ldwd=kd, workspace=wsh, workspace_bytes=nbh, route=stream,
                                                     taken=hrep), yh))
    if True:
        eager = []
        for _, fn, y in calls:
            fn()
            sync()
            eager.append(host(y, np.float32).copy())
        # the routes the test is about: selection in the staged row; staged X; the permute
        assert {"few_select", "few_xlds"} <= S.taken_names(S.route_taken(a)), S.taken_names(S.route_taken(a))
        assert {"few_xlds", "sparse_mma"} <= S.taken_names(S.route_taken(b))
        assert {"permute", "few_xlds"} <= S.taken_names(hrep.value)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            for _, fn, _ in calls:
                fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for _, fn, _ in calls:
                fn()
        torch.cuda.synchronize()
        for rep in range(3):
            for _, _, y in calls:
                y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for (label, _, y), ref in zip(calls, eager):
                assert np.array_equal(host(y, np.float32).view(np.uint32), ref.view(np.uint32)), f"{label} replay {rep}"
            for _, fn, _ in calls:   # eager work between the replays
                fn()
            sync()
        del g


# ---------------------------------------------- activation mitigations (PTS, VAR) ---

PTS_MODES = {"none": 0, "dyn": S.NM_PTS_DYNAMIC, "static": S.NM_PTS_STATIC, "var": S.NM_PTS_VAR,
             "dyn+var": S.NM_PTS_DYNAMIC | S.NM_PTS_VAR, "static+var": S.NM_PTS_STATIC | S.NM_PTS_VAR}


def pts_rows(rng, t, k):
    """Student-t rows shifted off zero, with an all-zero row, a row of few distinct values
    (ties after the shift) and a row spanning a wide dynamic range."""
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    xf = O.f32_from_bf16(x) + np.float32(0.3)
    x = synth.bf16_bits_from_f32(xf.astype(np.float32))
    if t >= 4:
        x[1] = 0
        x[2] = np.array([0x3F80, 0x4000, 0x3FC0, 0xBF80], np.uint16)[rng.integers(0, 4, size=k)]
        x[3, ::7] = 0x6000          # 2^65 (with fp8 weights the raw codes, up to 448, are summed
                                    # before the row scale: far larger values overflow fp32 there)
        x[3, 3::11] = 0x0005        # subnormal
    return x


def run_select_pts(x, n, m, mode, c=None, ld=None):
    t, k = x.shape
    y = empty((t, k), np.uint16, fill=-1)
    mask = empty((t, (k + 31) // 32), np.uint32, fill=-1)
    mu = empty((t,), np.float32, fill=float("nan"))
    al = empty((t,), np.float32, fill=float("nan"))
    S.nm_sparsify_pts(dev(x, ld), n, m, mode, y, mask, dev(c) if c is not None else None, mu, al, k=k, ldx=ld or k)
    sync()
    return host(y, np.uint16), host(mask, np.uint32), host(mu, np.float32), host(al, np.float32)


@pytest.mark.parametrize("mode", list(PTS_MODES))
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (4, 8), (8, 16), (5, 16), (16, 32), (31, 32)])
@pytest.mark.parametrize("t,k,pad", [(37, 1056, 0), (5, 8, 8), (300, 4096, 24)])
def test_select_pts_bitexact(mode, n, m, t, k, pad):
    """Shifted selection: S(x~), mask and the row means bit for bit; the variance factor
    within one fp32 rounding of the oracle's."""
    if k % m:
        pytest.skip("k not a multiple of m")
    print(f"select pts {mode} {n}:{m} t={t} k={k}", flush=True)
    rng = np.random.default_rng(t + k + m + n)
    x = pts_rows(rng, t, k)
    pts = PTS_MODES[mode]
    c = (rng.standard_normal(k) * 0.1).astype(np.float32) if pts & S.NM_PTS_STATIC else None
    y, mask, mu, al = run_select_pts(x, n, m, pts, c, ld=(k + pad) if pad else None)
    s_ref, keep, mu_ref, al_ref = O.sparsify_pts(x, n, m, pts, c)
    assert (y == s_ref).all(), "S(x~)"
    assert (mask == O.pack_mask(keep)).all(), "mask"
    if pts & S.NM_PTS_DYNAMIC:
        assert (mu.view(np.uint32) == mu_ref.view(np.uint32)).all(), "row means"
    if pts & S.NM_PTS_VAR:
        assert np.all(np.abs(al - al_ref) <= 2.0 ** -23 * np.abs(al_ref)), "variance factors"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("shifted", [False, True])
def test_weight_sums(kind, shifted):
    rng = np.random.default_rng(41)
    o, k = 300, 1056
    w = synth.normal_bf16(rng, (o, k), 0.02)
    c = (rng.standard_normal(k) * 0.1).astype(np.float32) if shifted else None
    out = empty((o,), np.float32, fill=float("nan"))
    if kind == "bf16":
        S.nm_weight_sums(dev(w), out, shift=dev(c) if c is not None else None)
        wv = O.bf16_to_f64(w)
    else:
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        S.nm_weight_sums(dev(q), out, S.NM_W_FP8E4M3, dev(sc), shift=dev(c) if c is not None else None)
        wv = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    sync()
    got = host(out, np.float32).astype(np.float64)
    ref = O.weight_sums(wv, c).astype(np.float64)
    absum = np.abs(wv) @ (np.abs(c.astype(np.float64)) if c is not None else np.ones(k))
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + k * 2.0 ** -50 * absum)


def check_pts(y, ref, s_bits, w_vals, alpha, beta, v, label=""):
    """Tolerance of a mitigated product: relative Frobenius <= 1e-3 and
    |err| <= 1e-2 * (alpha_t |S(x~)| |W|^T + |beta_t v_o|) + 1e-4."""
    y = np.asarray(y, np.float64)
    a = np.abs(O.bf16_to_f64(s_bits)) * (np.asarray(alpha, np.float64)[:, None] if alpha is not None else 1.0)
    bound = a @ np.abs(np.asarray(w_vals, np.float64)).T
    if v is not None:
        bb = np.abs(np.asarray(beta, np.float64))[:, None] if beta is not None else 1.0
        bound = bound + bb * np.abs(np.asarray(v, np.float64))[None, :]
    err = np.abs(y - ref)
    rel = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-3, f"{label}: relative Frobenius {rel:.3e}"
    worst = (err - 1e-2 * bound - 1e-4).max() if err.size else -1
    assert worst <= 0, f"{label}: per-element bound exceeded by {worst:.3e}"


def run_spmm_pts(x, w, n, m, pts, c=None, w8=None, s8=None, route=0):
    """One call: ACT_DYNAMIC with the mitigation; v from nm_weight_sums on the GPU."""
    t, k = x.shape
    o = (w if w is not None else w8).shape[0]
    wt, dt, sd = (dev(w), S.NM_W_BF16, None) if w8 is None else (dev(w8), S.NM_W_FP8E4M3, dev(s8))
    cd = dev(c) if c is not None else None
    v = None
    if pts & (S.NM_PTS_DYNAMIC | S.NM_PTS_STATIC):
        v = empty((o,), np.float32)
        S.nm_weight_sums(wt, v, dt, sd, shift=cd)
    y = empty((t, o), np.float32, fill=float("nan"))
    mask = empty((t, (k + 31) // 32), np.uint32, fill=-1)
    a = mk_args(S.NM_ACT_DYNAMIC, t, o, k, dev(x), wt, y, n=n, m=m, w_dtype=dt, w_scale=sd, x_mask_out=mask,
                pts=pts, pts_shift=cd, col_shift=v, route=route)
    nb = S.nm_spmm_workspace_size(a)
    ws = empty((max(nb, 16),), np.uint8)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nb
    spmm_call(a)
    sync()
    return host(y, np.float32), host(mask, np.uint32)


def pts_reference(x, w_bits, w_vals, n, m, pts, c, w8=None, s8=None):
    """The oracle's mitigated layer (v from the oracle's weight sums)."""
    v = O.weight_sums(w_vals, c) if pts & (S.NM_PTS_DYNAMIC | S.NM_PTS_STATIC) else None
    s, keep, mu, alpha = O.sparsify_pts(x, n, m, pts, c)
    if w8 is None:
        acc = O.gemm(s, w_bits)
    else:
        acc = O.spmm_act_fp8(s, w8, s8, m, m)          # n = m: S(x~) is already selected
    y = acc * (alpha.astype(np.float64)[:, None] if alpha is not None else 1.0)
    beta = None
    if v is not None:
        beta = mu if pts & S.NM_PTS_DYNAMIC else np.ones(x.shape[0], np.float32)
        y = y + beta.astype(np.float64)[:, None] * v.astype(np.float64)[None, :]
    return y, s, keep, alpha, beta, v


@pytest.mark.parametrize("mode", ["dyn", "static", "var", "dyn+var", "static+var"])
@pytest.mark.parametrize("t,route", [(1, ()), (1, ("few_stream",)), (16, ()), (64, ("few_tile",)),
                                     (64, ("few_stream",)), (128, ()), (300, ()), (600, ("tile_regs",)),
                                     (600, ())])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_spmm_pts_routes(mode, t, route, kind):
    """The mitigated layer in one call on every route that can take it (few-token streaming
    and split tile kernels with the reduction's epilogue, register and direct-to-LDS tile
    kernels): mask bit for bit, product within tolerance of the oracle."""
    print(f"spmm pts {mode} t={t} route={route} {kind}", flush=True)
    rng = np.random.default_rng(t + len(mode))
    o, k = 520, 2048
    x = pts_rows(rng, t, k)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    pts = PTS_MODES[mode]
    c = (rng.standard_normal(k) * 0.1).astype(np.float32) if pts & S.NM_PTS_STATIC else None
    if kind == "bf16":
        q = sc = None
        wv = O.bf16_to_f64(w)
    else:
        q, sc = synth.fp8_e4m3_quantize_rows(w)
        wv = O.fp8_e4m3_to_f64(q) * sc[:, None].astype(np.float64)
    for n, m in ((8, 16), (16, 32)):
        y, mask = run_spmm_pts(x, w if q is None else None, n, m, pts, c, q, sc, route=S.route_bits(*route))
        ref, s, keep, alpha, beta, v = pts_reference(x, w, wv, n, m, pts, c, q, sc)
        assert (mask == O.pack_mask(keep)).all()
        check_pts(y, ref, s, wv, alpha, beta, v, label=f"pts {mode} {n}:{m} t={t} {kind}")


def test_spmm_pts_two_pass_equals_one_call():
    """nm_sparsify_pts + ACT_MASKED with the caller's row terms gives the same bits as the
    one-call form (same kernels, same order)."""
    rng = np.random.default_rng(43)
    for t in (16, 128, 700):
        o, k = 264, 1024
        x = pts_rows(rng, t, k)
        w = synth.normal_bf16(rng, (o, k), 0.02)
        pts = S.NM_PTS_DYNAMIC | S.NM_PTS_VAR
        y1, _ = run_spmm_pts(x, w, 8, 16, pts)
        wd_ = dev(w)
        v = empty((o,), np.float32)
        S.nm_weight_sums(wd_, v)
        sx = empty((t, k), np.uint16)
        mu = empty((t,), np.float32)
        al = empty((t,), np.float32)
        S.nm_sparsify_pts(dev(x), 8, 16, pts, sx, None, None, mu, al)
        y2 = empty((t, o), np.float32, fill=float("nan"))
        a = mk_args(S.NM_ACT_MASKED, t, o, k, sx, wd_, y2, n=8, m=16, col_shift=v, row_shift=mu, row_scale=al)
        nb = S.nm_spmm_workspace_size(a)
        ws = empty((max(nb, 16),), np.uint8)
        a.workspace, a.workspace_bytes = ws.data_ptr(), nb
        spmm_call(a)
        sync()
        assert np.array_equal(y1.view(np.uint32), host(y2, np.float32).view(np.uint32)), f"t={t}"


@pytest.mark.parametrize("t", [128, 8192])
def test_spmm_pts_full_size(t, down_full):
    """The 8:16 down-projection (4096 x 14336) with D-PTS + VAR at 128 and 8192 tokens: the
    mask of every row bit for bit, every output written, the oracle on one row of every
    128-row band."""
    print(f"pts full t={t}", flush=True)
    x_all, w = down_full[0], down_full[1]
    x = x_all[:t]
    pts = S.NM_PTS_DYNAMIC | S.NM_PTS_VAR
    y, mask = run_spmm_pts(x, w, 8, 16, pts)
    assert np.isfinite(y).all(), "unwritten outputs"
    s_all, keep_all, mu_all, al_all = O.sparsify_pts(x, 8, 16, pts)
    assert (mask == O.pack_mask(keep_all)).all()
    rows = band_rows(t, 128, seed=t)
    wv = O.bf16_to_f64(w)
    ref, s, keep, alpha, beta, v = pts_reference(x[rows], w, wv, 8, 16, pts, None)
    check_pts(y[rows], ref, s, wv, alpha, beta, v, label=f"pts full t={t}")


@pytest.mark.parametrize("t", [64, 8192])
@pytest.mark.parametrize("name", ["qkv", "down"])
def test_spmm_pts_layer_full_size(layer8b, name, t):
    """Linears of the 8B-shaped layer (q|k|v 6144 x 4096, down 4096 x 14336) with D-PTS +
    VAR, 16:32 and 8:16, bf16 and fp8 weights: masks bit for bit on every row, every output
    written, the oracle on one row of every 256-row band (every 8 rows at 64 tokens)."""
    print(f"pts layer {name} t={t}", flush=True)
    parts = LAYER_GROUPS[name]
    st = synth.TRANSFORMER_SHAPES[parts[0]][2]
    x = layer8b["x"][st][:t]
    w = np.concatenate([layer8b["w"][p] for p in parts], 0)
    w8 = np.concatenate([layer8b["w8"][p] for p in parts], 0)
    s8 = np.concatenate([layer8b["s8"][p] for p in parts], 0)
    pts = S.NM_PTS_DYNAMIC | S.NM_PTS_VAR
    rows = band_rows(t, 256 if t > 256 else 8, seed=t)
    for n, m in ((16, 32), (8, 16)):
        s_all, keep_all, _, _ = O.sparsify_pts(x, n, m, pts)
        for kind in ("bf16", "fp8"):
            if kind == "bf16":
                y, mask = run_spmm_pts(x, w, n, m, pts)
                wv = O.bf16_to_f64(w)
                ref, s, keep, alpha, beta, v = pts_reference(x[rows], w, wv, n, m, pts, None)
            else:
                y, mask = run_spmm_pts(x, None, n, m, pts, None, w8, s8)
                wv = O.fp8_e4m3_to_f64(w8) * s8[:, None].astype(np.float64)
                ref, s, keep, alpha, beta, v = pts_reference(x[rows], w, wv, n, m, pts, None, w8, s8)
            assert (mask == O.pack_mask(keep_all)).all()
            assert np.isfinite(y).all(), "unwritten outputs"
            check_pts(y[rows], ref, s, wv, alpha, beta, v, label=f"pts layer {name} t={t} {n}:{m} {kind}")
