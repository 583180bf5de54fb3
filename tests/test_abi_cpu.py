"""C-ABI checks that need no GPU: the library loads, exports every function nm.h
declares, and rejects every malformed call with the documented status before any HIP
call is made.  Pointers here are fake, aligned or misaligned addresses that are never
dereferenced (validation fails first, or the call is a documented no-op)."""
import math
import os
import re
import subprocess

import pytest

import semi_structured_sparse_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 4096          # a fake, 16-byte aligned device address
Q = 8192
MIS = 4098        # misaligned


def declared_functions(header="nm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z0-9_]+)\s*\(", src)))


def exported_functions(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    return set(re.findall(r"\bT (nm_[a-z0-9_]+)", out))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"nm_sparsify", "nm_compress", "nm_lower_slide", "nm_spmm", "nm_hybrid_gemm"} <= set(names)
    exported = exported_functions(S.LIB_PATH)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = S.lib()
    for n in names:
        assert hasattr(L, n)
    # the measurement helpers are a library of their own, not part of the product's ABI
    from semi_structured_sparse_amd import probe
    pnames = declared_functions("nm_probe.h")
    assert pnames and not (set(pnames) & exported)
    assert set(pnames) <= exported_functions(probe.PROBE_LIB_PATH)


def test_library_reads_no_environment():
    """The boundary is stateless: routes come from the call's arguments, never from the
    process environment (the library imports no getenv / secure_getenv)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    assert not re.search(r"\b(secure_)?getenv\b", out), out


def test_route_fields_change_routes_not_results_host_side():
    """Route hints steer the workspace query (which is host arithmetic); the query never
    writes the caller's report."""
    a = spmm_args(t=64, o=4096, k=14336, n=8, m=16, ldx=14336, ldw=14336, ldy=4096)
    auto = S.nm_spmm_workspace_size(a)
    a.route = S.route_bits("no_few")
    no_few = S.nm_spmm_workspace_size(a)
    a.route = S.route_bits("few_stream")
    stream = S.nm_spmm_workspace_size(a)
    assert auto >= 64 * 14336 * 2 and no_few >= 64 * 14336 * 2
    assert auto != stream            # the split tile route and the streaming route need different scratch
    assert S.route_taken(a) == 0
    assert set(S.ROUTE.values()) == {1 << i for i in range(15)}
    assert set(S.TAKEN.values()) == {1 << i for i in range(18)}
    # the header's values are the binding's
    src = open(os.path.join(ROOT, "include", "nm.h")).read()
    for name, bit in S.ROUTE.items():
        i = int(math.log2(bit))
        assert re.search(rf"NM_ROUTE_{name.upper()} = 1u << {i}\b", src), name
    for name, bit in S.TAKEN.items():
        i = int(math.log2(bit))
        assert re.search(rf"NM_TAKEN_{name.upper()} = 1u << {i}\b", src), name


def test_mid_range_workspace_holds_the_split_partials():
    """Above 128 tokens, a product whose 256 x 256 output tiles number under 128 takes the
    split tile kernel: the workspace query adds its partial tiles (splits x t x o fp32,
    splits = 256 // 128-row tiles, at most half the K-steps) after the staging; the
    no_few and tile hints keep the large-tile kernels and ask for no partials."""
    t, o, k = 300, 4096, 14336
    a = spmm_args(t=t, o=o, k=k, n=8, m=16, ldx=k, ldw=k, ldy=o)
    stage = -(-(t * k * 2 + 64) // 256) * 256
    splits = 256 // (32 * 3)
    assert S.nm_spmm_workspace_size(a) == stage + splits * t * o * 4
    for hint in ("no_few", "tile_lds", "tile_regs"):
        a.route = S.route_bits(hint)
        assert S.nm_spmm_workspace_size(a) == t * k * 2 + 64, hint
    # enough large tiles: no partials
    a = spmm_args(t=4096, o=o, k=k, n=8, m=16, ldx=k, ldw=k, ldy=o)
    assert S.nm_spmm_workspace_size(a) == 4096 * k * 2 + 64


def test_large_tile_split_workspace():
    """256 x 256 tiles that fill under one round, with at least 100 K-steps of 64 per range
    (dense): the reduction splits in 256 // tiles ranges, whose partial tiles the workspace
    query adds, unless 256 x 128 tiles fill three quarters to one round (then those,
    unsplit); fewer steps per range take the 128-row split kernel instead."""
    k = 14336
    def size(t, o=4096, **kw):
        return S.nm_spmm_workspace_size(spmm_args(mode=S.NM_ACT_MASKED, t=t, o=o, k=k, ldx=k, ldw=k, ldy=o, **kw))
    assert size(2500, o=2056) == 2 * 2500 * 2056 * 4   # 90 tiles, two ranges of 112 steps (180 half tiles)
    assert size(2048) == 0                         # 128 tiles, but 256 half tiles fill one round
    assert size(1536) == 0                         # 96 tiles, 192 half tiles
    assert size(1024) == 0                         # 64 tiles: four ranges of 56 steps are too short;
                                                   # 256 tiles of 128 rows, unsplit
    assert size(3072) == 0                         # 192 tiles: one round already
    assert size(2500, o=2056, route=S.route_bits("tile_lds")) == 0


def test_status_strings_and_version():
    for code in range(7):
        assert S.nm_status_str(code).startswith("NM_")
    assert S.nm_status_str(S.NM_ESCRATCH).startswith("NM_ESCRATCH")
    assert S.nm_version() >= 100


def st(fn, *a, **kw):
    return fn(*a, check=False, stream=0, **kw)


def test_sparsify_validation():
    f = S.nm_sparsify
    assert st(f, P, 2, 4, y=None, mask=None, rows=4, k=8, ldx=8, ldy=8) == S.NM_EINVAL       # no output
    assert st(f, None, 2, 4, y=Q, rows=4, k=8, ldx=8, ldy=8) == S.NM_EINVAL                   # null x
    assert st(f, P, 0, 4, y=Q, rows=4, k=8, ldx=8, ldy=8) == S.NM_EINVAL                      # n < 1
    assert st(f, P, 5, 4, y=Q, rows=4, k=8, ldx=8, ldy=8) == S.NM_EINVAL                      # n > m
    assert st(f, P, 2, 7, y=Q, rows=4, k=14, ldx=16, ldy=16) == S.NM_EUNSUPPORTED             # m = 7
    assert st(f, P, 2, 6, y=Q, mask=Q, rows=4, k=12, ldx=16, ldy=16) == S.NM_EUNSUPPORTED     # m = 6 mask
    assert st(f, P, 2, 6, y=Q, rows=4, k=10, ldx=16, ldy=16) == S.NM_ESHAPE                   # k % 6
    assert st(f, P, 2, 6, y=Q, rows=4, k=12, ldx=13, ldy=16) == S.NM_EALIGN                   # ld odd (m=6)
    assert st(f, P, 7, 6, y=Q, rows=4, k=12, ldx=16, ldy=16) == S.NM_EINVAL                   # n > m (m=6)
    assert st(f, P, 4, 10, y=Q, mask=Q, rows=4, k=20, ldx=20, ldy=20) == S.NM_EUNSUPPORTED    # m = 10 mask
    assert st(f, P, 2, 4, y=Q, rows=4, k=10, ldx=16, ldy=16) == S.NM_ESHAPE                   # k % m
    assert st(f, P, 2, 4, y=Q, rows=4, k=16, ldx=8, ldy=16) == S.NM_ESHAPE                    # ldx < k
    assert st(f, P, 2, 4, y=Q, rows=-1, k=16, ldx=16, ldy=16) == S.NM_ESHAPE                  # rows < 0
    assert st(f, MIS, 2, 4, y=Q, rows=4, k=16, ldx=16, ldy=16) == S.NM_EALIGN                 # pointer
    assert st(f, P, 4, 8, y=Q, rows=4, k=16, ldx=20, ldy=16) == S.NM_EALIGN                   # ld % 8
    assert st(f, P, 2, 4, y=Q, rows=4, k=16, ldx=18, ldy=16) == S.NM_EALIGN                   # ld % 4 (m=4)
    assert st(f, P, 2, 4, y=None, mask=MIS, rows=4, k=16, ldx=16, ldy=0) == S.NM_EALIGN
    assert st(f, P, 2, 4, y=Q, rows=1 << 62, k=16, ldx=16, ldy=16) == S.NM_ESHAPE             # overflow
    assert st(f, P, 2, 4, y=Q, rows=0, k=16, ldx=16, ldy=16) == S.NM_OK                       # empty: no-op
    assert st(f, P, 2, 4, y=Q, rows=3, k=0, ldx=0, ldy=0) == S.NM_OK


def test_compress_decompress_validation():
    c = S.nm_compress
    assert st(c, P, 4, 8, Q, Q, S.NM_META_2BIT, rows=2, k=16, ldx=16) == S.NM_EINVAL          # 2bit needs 2:4
    assert st(c, P, 2, 4, None, Q, S.NM_META_U8, rows=2, k=16, ldx=16) == S.NM_EINVAL         # null values
    assert st(c, P, 2, 4, Q, Q, 7, rows=2, k=16, ldx=16) == S.NM_EINVAL                       # bad fmt
    assert st(c, P, 2, 4, Q + 2, Q, S.NM_META_U8, rows=2, k=16, ldx=16) == S.NM_EALIGN
    d = S.nm_decompress
    assert st(d, P, Q, S.NM_META_2BIT, 2, 16, 4, 8, Q, ldy=16) == S.NM_EINVAL
    assert st(d, P, Q, S.NM_META_U8, 2, 16, 2, 4, None, ldy=16) == S.NM_EINVAL
    assert st(d, P, Q, S.NM_META_U8, 2, 18, 2, 4, Q, ldy=24) == S.NM_ESHAPE


def test_slide_validation():
    f = S.nm_lower_slide
    assert st(f, P, P, 4, 16, 1, Q, Q, S.NM_META_2BIT) == S.NM_EINVAL                         # N < 2
    assert st(f, P, P, 4, 18 * 2, 9, Q, Q, S.NM_META_2BIT) == S.NM_EUNSUPPORTED               # N > 8
    assert st(f, P, P, 4, 12, 4, Q, Q, S.NM_META_2BIT) == S.NM_ESHAPE                         # k % 2N
    assert st(f, None, P, 4, 16, 4, Q, Q, S.NM_META_2BIT) == S.NM_EINVAL
    assert st(f, P, P, 4, 16, 4, Q, Q, 3) == S.NM_EINVAL
    g = S.nm_slide_lift
    assert st(g, P, 4, Q, t=2, k=16, ldx=16, ldo=8) == S.NM_ESHAPE                           # ldo < K'
    assert st(g, P + 8, 4, Q, t=2, k=16, ldx=16, ldo=24) == S.NM_EALIGN
    assert st(g, P, 4, None, t=2, k=16, ldx=16, ldo=24) == S.NM_EINVAL


def spmm_args(**kw):
    base = dict(mode=S.NM_ACT_DYNAMIC, t=4, o=8, k=16, x=P, w=Q, y=P + 1024, n=2, m=4, ldx=16, ldw=16, ldy=8)
    base.update(kw)
    mode, t, o, k, x, w, y = (base.pop(key) for key in ("mode", "t", "o", "k", "x", "w", "y"))
    return S.make_spmm_args(mode, t, o, k, x, w, y, **base)


def test_spmm_validation():
    f = lambda a: S.nm_spmm(a, check=False, stream=0)  # noqa: E731
    assert S.lib().nm_spmm(None, None) == S.NM_EINVAL
    assert f(spmm_args(mode=9)) == S.NM_EINVAL
    assert f(spmm_args(y=None)) == S.NM_EINVAL
    assert f(spmm_args(ldy=4)) == S.NM_ESHAPE                         # ldy < o
    assert f(spmm_args(y=P + 1028)) == S.NM_EALIGN                    # y not 16-byte aligned
    assert f(spmm_args(accumulate=2)) == S.NM_EINVAL
    assert f(spmm_args(k=18)) == S.NM_ESHAPE                          # k % m
    assert f(spmm_args(n=9, m=8)) == S.NM_EINVAL
    assert f(spmm_args(w_dtype=S.NM_W_FP8E4M3, w_scale=None)) == S.NM_EINVAL   # fp8 needs scales
    assert f(spmm_args(w_dtype=S.NM_W_FP8E4M3, w_scale=P, ldw=24)) == S.NM_EALIGN
    assert f(spmm_args(x=MIS)) == S.NM_EALIGN
    assert f(spmm_args(mode=S.NM_W_COMPRESSED, w_meta=P, w_meta_fmt=S.NM_META_U8)) == S.NM_EUNSUPPORTED
    assert f(spmm_args(mode=S.NM_W_COMPRESSED, w_meta=None, w_meta_fmt=S.NM_META_2BIT)) == S.NM_EINVAL
    assert f(spmm_args(mode=S.NM_W_SLIDE, ns=4, k=12, w_meta=P)) == S.NM_ESHAPE
    assert f(spmm_args(mode=S.NM_W_SLIDE, ns=1, w_meta=P)) == S.NM_EINVAL
    assert f(spmm_args(mode=S.NM_ACT_COMPRESSED, x_meta=None)) == S.NM_EINVAL
    assert f(spmm_args(mode=S.NM_ACT_COMPRESSED, x_meta=P, x_meta_fmt=S.NM_META_2BIT, n=4, m=8)) == S.NM_EINVAL
    assert f(spmm_args(t=0)) == S.NM_OK                                # empty: no-op
    a = spmm_args(t=64, k=4096)
    assert S.nm_spmm_workspace_size(a) >= 64 * 2048 * 2 + 64 * 512
    a = spmm_args(t=64, k=4096, n=8, m=16)
    assert S.nm_spmm_workspace_size(a) >= 64 * 4096 * 2
    # few tokens, few output rows: the reduction is split across workgroups and the
    # partial sums need scratch; many output rows need none
    a = spmm_args(mode=S.NM_W_COMPRESSED, t=4, o=64, k=4096, w_meta=P, w_meta_fmt=S.NM_META_2BIT)
    assert S.nm_spmm_workspace_size(a) >= 2 * 4 * 64 * 4
    a = spmm_args(mode=S.NM_W_COMPRESSED, t=4, o=8192, k=4096, w_meta=P, w_meta_fmt=S.NM_META_2BIT, ldy=8192)
    assert S.nm_spmm_workspace_size(a) == 0
    # large tokens: the K-blocked copy of the weight positions (2:4); 6:8 lowered to 2:4
    # over K' = 1.5 K: the direct-to-LDS kernel lifts X in its loads, so the positions
    # alone, and with the lift_copy hint the lifted X before them
    a = spmm_args(mode=S.NM_W_COMPRESSED, t=4096, o=4096, k=6144, w_meta=P, w_meta_fmt=S.NM_META_2BIT, ldx=6144,
                  ldy=4096)
    assert S.nm_spmm_workspace_size(a) >= 4096 * 6144 // 8
    a = spmm_args(mode=S.NM_W_SLIDE, ns=4, t=4096, o=4096, k=4096, w_meta=P, w_meta_fmt=S.NM_META_2BIT, ldx=4096,
                  ldy=4096)
    assert S.nm_spmm_workspace_size(a) == 4096 * 6144 // 8
    a.route = S.route_bits("lift_copy")
    assert S.nm_spmm_workspace_size(a) >= 4096 * 6144 * 2 + 4096 * 6144 // 8
    a = spmm_args(mode=S.NM_W_COMPRESSED, t=4, o=8, k=16, w_meta=P, w_meta_fmt=S.NM_META_2BIT,
                  workspace=MIS, workspace_bytes=1 << 20)
    assert f(a) == S.NM_EALIGN


def test_sparsify_scored_validation():
    f = lambda *a, **kw: S.nm_sparsify_scored(*a, check=False, stream=0, **kw)  # noqa: E731
    x = dict(rows=4, k=16, ldx=16, ldy=16)
    assert f(P, 3, 6, Q, 0, P, None, rows=4, k=12, ldx=16, ldy=16) == S.NM_EUNSUPPORTED    # width 6
    assert f(P, 0, 4, Q, 0, P, None, **x) == S.NM_EINVAL                                  # n < 1
    assert f(P, 5, 4, Q, 0, P, None, **x) == S.NM_EINVAL                                  # n > m
    assert f(P, 2, 4, Q, 2, P, None, **x) == S.NM_EINVAL                                  # mode
    assert f(P, 2, 4, Q, 0, None, None, **x) == S.NM_EINVAL                               # no output
    assert f(P, 2, 4, None, 0, P, None, **x) == S.NM_EINVAL                               # no scores
    assert f(P, 2, 4, MIS, 0, P, None, **x) == S.NM_EALIGN                                # scores aligned
    assert f(P, 2, 4, Q, 0, None, MIS, **x) == S.NM_EALIGN                                # mask aligned
    assert f(P, 2, 8, Q, 0, P, None, rows=4, k=12, ldx=16, ldy=16) == S.NM_ESHAPE          # k % m
    assert f(P, 2, 4, Q, 0, P, None, rows=4, k=16, ldx=8, ldy=16) == S.NM_ESHAPE           # ldx < k
    assert f(P, 2, 4, Q, 0, P, None, rows=0, k=16, ldx=16, ldy=16) == S.NM_OK             # empty: no-op


def test_w8a8_validation():
    q = lambda *a, **kw: S.nm_quant_lift(*a, check=False, stream=0, **kw)  # noqa: E731
    assert q(P, 1, Q, P, t=4, k=16, ldx=16, ldq=32) == S.NM_EINVAL                 # ns < 2
    assert q(P, 9, Q, P, t=4, k=18, ldx=18, ldq=32) == S.NM_EUNSUPPORTED           # ns > 8
    assert q(P, 4, Q, P, t=4, k=12, ldx=16, ldq=32) == S.NM_ESHAPE                 # k % 2ns
    assert q(P, 4, Q, P, t=4, k=16, ldx=16, ldq=16) == S.NM_ESHAPE                 # ldq < K' (24)
    assert q(P, 4, Q, P, t=4, k=16, ldx=16, ldq=40) == S.NM_EALIGN                 # ldq % 16
    assert q(P, 4, None, P, t=4, k=16, ldx=16, ldq=32) == S.NM_EINVAL              # no codes
    assert q(P, 4, Q, P, t=0, k=16, ldx=16, ldq=32) == S.NM_OK                     # empty
    f = lambda a: S.nm_spmm(a, check=False, stream=0)  # noqa: E731
    w8 = dict(mode=S.NM_W_SLIDE, ns=4, w_dtype=S.NM_W_FP8E4M3, w_meta=P, w_meta_fmt=S.NM_META_2BIT)
    assert f(spmm_args(k=256, ldx=256, w_scale=None, **w8)) == S.NM_EINVAL         # fp8 needs scales
    assert f(spmm_args(k=64, ldx=64, w_scale=P, **w8)) == S.NM_EUNSUPPORTED         # K' = 96 not % 128
    assert f(spmm_args(k=256, ldx=256, w_scale=P, **w8)) == S.NM_EINVAL             # needs the workspace
    a = spmm_args(t=4096, o=4096, k=4096, ldx=4096, ldy=4096, w_scale=P, **w8)
    assert S.nm_spmm_workspace_size(a) >= 4096 * 6144 + 4096 * 4 + 4096 * 6144 // 8


def test_spense_validation():
    g = lambda *a, **kw: S.nm_spense_glu_order(*a, check=False, stream=0, **kw)  # noqa: E731
    dims = dict(hidden=16, inter=32, ld_gu=16, ld_d=32, workspace_bytes=1 << 20)
    assert g(P, P, Q, Q, Q, 4, 2, P, Q, **dims) == S.NM_EINVAL                     # strategy
    assert g(P, P, Q, Q, Q, 40, 0, P, Q, **dims) == S.NM_ESHAPE                    # n_dense > inter
    assert g(P, P, Q, Q, Q, 4, 0, None, Q, **dims) == S.NM_EINVAL                  # no perm
    assert g(P, P, Q, Q, Q, 4, 0, P, None, **dims) == S.NM_EINVAL                  # no workspace
    assert g(P, P, Q, Q, Q, 4, 0, P, Q, hidden=16, inter=32, ld_gu=16, ld_d=32,
             workspace_bytes=100) == S.NM_EINVAL                                    # workspace too small
    assert g(None, P, Q, Q, Q, 4, 0, P, Q, **dims) == S.NM_EINVAL                  # loss scores need weights
    assert g(P, P, Q, None, Q, 4, 0, P, Q, **dims) == S.NM_EINVAL                  # ... and hs_in
    assert g(P, P, Q, Q, Q, 4, 0, MIS, Q, **dims) == S.NM_EALIGN
    assert g(None, None, None, None, None, 0, S.NM_SPENSE_TAIL, P, Q, hidden=0, inter=0, ld_gu=0, ld_d=0,
             workspace_bytes=0) == S.NM_OK                                          # empty
    assert S.nm_spense_glu_order_workspace_size(14336) >= 14336 * 12
    k = lambda *a, **kw: S.nm_spense_pack(*a, check=False, stream=0, **kw)  # noqa: E731
    pk = dict(o=16, k=32, ldw=32, ldwd=32, workspace_bytes=1 << 20)
    assert k(P, 2, Q, 8, P, Q, S.NM_META_2BIT, P, Q, **pk) == S.NM_EINVAL          # axis
    assert k(P, 0, Q, 8, P, Q, 7, P, Q, **pk) == S.NM_EINVAL                       # meta format
    assert k(P, 0, Q, 20, P, Q, S.NM_META_2BIT, P, Q, **pk) == S.NM_ESHAPE         # n_sparse > o
    assert k(P, 1, Q, 6, P, Q, S.NM_META_2BIT, P, Q, **pk) == S.NM_ESHAPE          # n_sparse % 4 (columns)
    assert k(P, 0, Q, 8, P, Q, S.NM_META_2BIT, P, Q, o=16, k=30, ldw=32, ldwd=32,
             workspace_bytes=1 << 20) == S.NM_ESHAPE                                # k % 4 (rows)
    assert k(P, 0, None, 8, P, Q, S.NM_META_2BIT, P, Q, **pk) == S.NM_EINVAL       # no perm
    assert k(P, 0, Q, 8, P, Q, S.NM_META_2BIT, P, None, o=16, k=32, ldw=32, ldwd=32,
             workspace_bytes=0) == S.NM_EINVAL                                      # rows need the workspace
    assert k(P, 0, MIS, 8, P, Q, S.NM_META_2BIT, P, Q, **pk) == S.NM_EALIGN
    assert S.nm_spense_pack_workspace_size(16, 32, 0, 8) >= 8 * 32 * 2
    assert S.nm_spense_pack_workspace_size(16, 32, 1, 8) == 0
    f = lambda *a, **kw: S.nm_spense_outsplit_gemm(*a, check=False, stream=0, **kw)  # noqa: E731
    od = dict(t=4, k=32, ldx=32, ldwd=32, ldy=64)
    assert f(P, Q, Q, 32, Q, 32, P, **dict(od, k=30)) == S.NM_ESHAPE                # k % 4
    assert f(P, Q, Q, 32, Q, 40, P, **od) == S.NM_ESHAPE                            # ldy < o_s + o_d
    assert f(P, Q, Q, 30, Q, 32, P, **dict(od, ldy=64)) == S.NM_EALIGN              # o_s % 4
    assert f(P, Q, Q, 32, Q, 32, P, **dict(od, t=0)) == S.NM_OK                     # empty
    assert S.nm_spense_outsplit_workspace_size(64, 4096, 21504, 7168) > 0


def test_hybrid_validation():
    g = lambda *a, **kw: S.nm_hybrid_gemm(*a, check=False, stream=0, **kw)  # noqa: E731
    assert g(P, P, 6, P, 2, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_ESHAPE  # k_s % 4
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_U8, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EUNSUPPORTED
    assert g(P, None, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EINVAL
    assert g(P, None, 12, None, 4, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EALIGN
    assert g(P, P, 8, P, 8, None, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EINVAL
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, None, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EINVAL
    # gathered form: the permuted-X staging must fit in the workspace
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8) == S.NM_EINVAL
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8, workspace=Q,
             workspace_bytes=4 * 16 * 2 - 1) == S.NM_EINVAL
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=16, ldwd=8, ldy=8, workspace=MIS,
             workspace_bytes=1 << 20) == S.NM_EALIGN
    assert g(P, P, 8, P, 8, Q, Q, S.NM_META_2BIT, Q, 8, P, t=4, ldx=8, ldwd=8, ldy=8, workspace=Q,
             workspace_bytes=1 << 20) == S.NM_ESHAPE                                      # ldx < k_s + k_d
    assert S.nm_hybrid_gemm_workspace_size(4, 8, 8, 8, True) >= 4 * 16 * 2
    assert S.nm_hybrid_gemm_workspace_size(4, 8, 8, 14336, False) == 0
    assert S.nm_hybrid_gemm_workspace_size(0, 8, 8, 8, True) == 0
    # large-token hybrid: permuted X, then the K-blocked copy of the 2:4 positions
    assert S.nm_hybrid_gemm_workspace_size(2048, 3072, 1024, 14336, True) >= 2048 * 4096 * 2 + 14336 * 3072 // 8
    assert S.nm_hybrid_gemm_workspace_size(2048, 3072, 1024, 14336, False) >= 14336 * 3072 // 8
    p = lambda *a, **kw: S.nm_hybrid_pack(*a, check=False, stream=0, **kw)  # noqa: E731
    assert S.nm_hybrid_pack_workspace_size(4096) >= 4096 * 12
    assert p(P, 20, P, P, Q, Q, S.NM_META_2BIT, Q, P, o=8, k=16, ldw=16, ldwd=16, workspace_bytes=1 << 20) == S.NM_ESHAPE
    assert p(P, 6, P, P, Q, Q, S.NM_META_2BIT, Q, P, o=8, k=16, ldw=16, ldwd=8, workspace_bytes=1 << 20) == S.NM_ESHAPE
    assert p(P, 4, P, P, Q, Q, S.NM_META_2BIT, Q, P, o=8, k=16, ldw=16, ldwd=8, workspace_bytes=16) == S.NM_EINVAL
    assert p(P, 4, P, P, Q, Q, S.NM_META_2BIT, Q, None, o=8, k=16, ldw=16, ldwd=8, workspace_bytes=1 << 20) == S.NM_EINVAL
    assert p(P, 4, P, P, Q, Q, 5, Q, P, o=8, k=16, ldw=16, ldwd=8, workspace_bytes=1 << 20) == S.NM_EINVAL


def test_binding_lowered_k_matches_oracle():
    import oracle as O
    for ns in range(2, 9):
        for k in (2 * ns, 2 * ns * 7, 4096 - 4096 % (2 * ns)):
            assert S.lowered_k(k, ns) == O.lowered_k(k, ns)



def test_probe_helpers_host_side():
    """Measurement helpers: sizes are host arithmetic; bad arguments are rejected before
    any GPU call."""
    from semi_structured_sparse_amd import probe as P_
    assert P_.nm_probe_sink_bytes() >= 2048 * 256 * 4
    assert P_.nm_probe_mfma_flops(10) == 1024 * 4 * 16 * 10 * 16 * 16 * 32 * 2
    assert P_.nm_probe_mfma_flops(-1) == 0
    assert P_.nm_probe_read(None, -16, None, check=False, stream=0) == S.NM_ESHAPE
    assert P_.nm_probe_read(None, 24, None, check=False, stream=0) == S.NM_ESHAPE
    assert P_.nm_probe_read(None, 32, None, check=False, stream=0) == S.NM_EINVAL
    assert P_.nm_probe_read(16 * 1024 + 4, 32, 16 * 1024, check=False, stream=0) == S.NM_EALIGN
    assert P_.nm_probe_read(16 * 1024, 32, 16 * 1024, mode=3, check=False, stream=0) == S.NM_EINVAL
    assert P_.nm_probe_read(16 * 1024, 32, 16 * 1024, mode=2, check=False, stream=0) == S.NM_ESHAPE
    assert P_.nm_probe_mfma(-1, 16 * 1024, check=False, stream=0) == S.NM_ESHAPE
    assert P_.nm_probe_mfma(1, None, check=False, stream=0) == S.NM_EINVAL
    assert P_.nm_probe_mfma(1, 16 * 1024 + 8, check=False, stream=0) == S.NM_EALIGN


def test_pts_validation():
    f = lambda *a, **kw: S.nm_sparsify_pts(*a, check=False, stream=0, **kw)  # noqa: E731
    d = dict(rows=4, k=16, ldx=16, ldy=16)
    assert f(P, 8, 16, 8, Q, **d) == S.NM_EINVAL                                  # unknown mode bit
    assert f(P, 8, 16, 3, Q, shift=Q, **d) == S.NM_EINVAL                         # two shifts
    assert f(P, 8, 16, S.NM_PTS_STATIC, Q, **d) == S.NM_EINVAL                    # static needs the shift
    assert f(P, 8, 16, S.NM_PTS_VAR, Q, **d) == S.NM_EINVAL                       # VAR needs row_scale
    assert f(P, 8, 16, 0, None, **d) == S.NM_EINVAL                               # S(x~) required
    assert f(P, 2, 4, 1, Q, rows=4, k=12, ldx=16, ldy=16) == S.NM_ESHAPE          # k % 8
    assert f(P, 3, 6, 1, Q, rows=4, k=12, ldx=16, ldy=16) == S.NM_EUNSUPPORTED    # width 6
    assert f(P, 8, 16, 1, Q, mask=MIS, **d) == S.NM_EALIGN
    assert f(P, 8, 16, 1, Q, row_shift=MIS, **d) == S.NM_EALIGN
    assert f(P, 8, 16, 1, Q, rows=0, k=16, ldx=16, ldy=16) == S.NM_OK             # empty
    g = lambda *a, **kw: S.nm_weight_sums(*a, check=False, stream=0, **kw)  # noqa: E731
    assert g(P, Q, 7, o=4, k=16, ldw=16) == S.NM_EINVAL                            # dtype
    assert g(P, Q, S.NM_W_FP8E4M3, None, o=4, k=16, ldw=16) == S.NM_EINVAL         # fp8 needs scales
    assert g(P, None, o=4, k=16, ldw=16) == S.NM_EINVAL                            # output
    assert g(P, Q, o=4, k=16, ldw=8) == S.NM_ESHAPE
    assert g(P, Q + 4, o=4, k=16, ldw=16) == S.NM_EALIGN
    f2 = lambda a: S.nm_spmm(a, check=False, stream=0)  # noqa: E731
    base = dict(t=4, o=8, k=16, n=8, m=16)
    assert f2(spmm_args(pts=S.NM_PTS_DYNAMIC, **base)) == S.NM_EINVAL             # shift needs col_shift
    assert f2(spmm_args(pts=S.NM_PTS_DYNAMIC, col_shift=Q, **base)) == S.NM_EINVAL  # needs the workspace
    assert f2(spmm_args(pts=S.NM_PTS_VAR, col_shift=Q, **base)) == S.NM_EINVAL      # no shift, no col_shift
    assert f2(spmm_args(pts=S.NM_PTS_VAR, row_scale=Q, **base)) == S.NM_EINVAL      # rows terms: masked only
    assert f2(spmm_args(mode=S.NM_ACT_MASKED, pts=S.NM_PTS_VAR, **base)) == S.NM_EINVAL
    assert f2(spmm_args(mode=S.NM_ACT_MASKED, row_shift=Q, **base)) == S.NM_EINVAL  # row_shift needs col_shift
    assert f2(spmm_args(mode=S.NM_ACT_MASKED, row_scale=MIS, **base)) == S.NM_EALIGN
    assert f2(spmm_args(mode=S.NM_W_COMPRESSED, w_meta=P, w_meta_fmt=S.NM_META_2BIT, row_scale=Q)) == \
        S.NM_EUNSUPPORTED
    assert f2(spmm_args(pts=S.NM_PTS_VAR, t=4, o=8, k=20, n=2, m=4, ldx=24, ldw=24)) == S.NM_ESHAPE  # k % 8
    a = spmm_args(pts=S.NM_PTS_DYNAMIC | S.NM_PTS_VAR, col_shift=Q, t=64, o=4096, k=14336, ldx=14336,
                  ldw=14336, ldy=4096, n=8, m=16)
    assert S.nm_spmm_workspace_size(a) >= 64 * 14336 * 2 + 2 * 64 * 4


def test_noalloc_validation():
    """The no-allocation entry point rejects a caller workspace and, before any HIP call, a
    call whose scratch need exceeds its buffer."""
    f = lambda a: S.nm_spmm_noalloc(a, check=False, stream=0)  # noqa: E731
    assert S.lib().nm_spmm_noalloc(None, None) == S.NM_EINVAL
    assert f(spmm_args(workspace=Q, workspace_bytes=1024)) == S.NM_EINVAL
    big = spmm_args(t=8192, o=4096, k=14336, ldx=14336, ldw=14336, ldy=4096, n=8, m=16)
    assert S.nm_spmm_workspace_size(big) > S.NM_NOALLOC_SCRATCH_BYTES
    assert f(big) == S.NM_ESCRATCH
    assert f(spmm_args(accumulate=2)) == S.NM_EINVAL          # the usual validation still applies
