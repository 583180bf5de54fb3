"""Pins of the CPU oracle against facts that do not come from the oracle itself:
the pages' printed figures, hand-worked examples, brute force over tiny inputs,
exact rational arithmetic, closed forms and an independent library (torch's fp8)."""
import json
import math
import os
import struct
from fractions import Fraction
from itertools import combinations, product

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bits_of(v):
    """Python float / "-0" -> bf16 bits (values in the fixtures are exact in bf16)."""
    if v == "-0":
        return 0x8000
    return struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16


def value_of(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def arr(rows):
    return np.array([[bits_of(v) for v in r] for r in rows], dtype=np.uint16)


# ------------------------------------------------------------------ brute force ---

def brute_keep(group_vals, n):
    """Independent definition: among all n-subsets (lexicographic order) take the first
    one with the largest sum of |x|.  Equals top-n by magnitude with ties to the lower
    index (the lexicographically smallest tuple takes the lowest-index ties)."""
    best, best_sum = None, None
    for comb in combinations(range(len(group_vals)), n):
        s = sum(abs(Fraction(group_vals[i])) for i in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    keep = [False] * len(group_vals)
    for i in best:
        keep[i] = True
    return keep


ALPHABET = [0x0000, 0x8000, 0x3F00, 0xBF00, 0x3F80, 0xBF80, 0x4000, 0xC000]  # 0,-0,.5,-.5,1,-1,2,-2


def test_select_bruteforce_all_2of4_alphabet_groups():
    groups = np.array(list(product(ALPHABET, repeat=4)), dtype=np.uint16)   # 4096 groups
    vals = [[value_of(b) for b in g] for g in groups]
    for n in range(1, 5):
        keep = O.select_keep(groups, n, 4)
        for gi in range(len(groups)):
            assert list(keep[gi]) == brute_keep(vals[gi], n), (n, groups[gi])


def test_select_bruteforce_m8_three_magnitudes():
    mags = [0x0000, 0x3F80, 0x4000]      # 0, 1, 2 -> many ties
    rng = np.random.default_rng(11)
    groups = np.array(list(product(mags, repeat=8)), dtype=np.uint16)        # 6561 groups
    signs = rng.integers(0, 2, size=groups.shape).astype(np.uint16) << np.uint16(15)
    groups = groups | signs
    vals = [[value_of(b) for b in g] for g in groups]
    for n in (1, 3, 4, 6, 7):
        keep = O.select_keep(groups, n, 8)
        for gi in range(0, len(groups), 3):
            assert list(keep[gi]) == brute_keep(vals[gi], n)


def test_select_bruteforce_m16_random_ties():
    rng = np.random.default_rng(12)
    g = rng.choice(np.array(ALPHABET, dtype=np.uint16), size=(12, 16))
    vals = [[value_of(b) for b in row] for row in g]
    for n in (4, 8, 12):
        keep = O.select_keep(g, n, 16)
        for gi in range(len(g)):
            assert list(keep[gi]) == brute_keep(vals[gi], n)


def _certificate(vals_bits, keep_row, n):
    """Exchange certificate: exactly n kept and every kept i precedes every pruned j in
    the order (|x| descending, index ascending)."""
    mags = [abs(value_of(b)) if not math.isnan(value_of(b)) else math.inf for b in vals_bits]
    kept = [i for i, k in enumerate(keep_row) if k]
    pruned = [j for j, k in enumerate(keep_row) if not k]
    assert len(kept) == n
    for i in kept:
        for j in pruned:
            assert mags[i] > mags[j] or (mags[i] == mags[j] and i < j)


def test_select_certificate_m32_and_all_n():
    rng = np.random.default_rng(13)
    x = synth.student_t_bf16(rng, (6, 32 * 8), 4.0, 0.5)
    x[0, :32] = 0x3F80                   # a fully tied group
    x[1, 32:64] = rng.choice(np.array(ALPHABET, np.uint16), size=32)
    for m in (4, 8, 16, 32):
        for n in sorted({1, m // 4 or 1, m // 2, m - 1, m}):
            keep = O.select_keep(x, n, m)
            for r in range(x.shape[0]):
                for g in range(x.shape[1] // m):
                    _certificate(x[r, g * m:(g + 1) * m], keep[r, g * m:(g + 1) * m], n)


def test_select_special_values():
    # subnormal < smallest normal; inf beats finite; NaN ranks above inf (policy); +0 == -0
    sub, norm, inf, nan = 0x0001, 0x0080, 0x7F80, 0x7FC0
    g = np.array([[sub, norm, 0x8000, 0x0000],
                  [0x4000, inf | 0x8000, 0x3F80, 0x0000],
                  [inf, 0x3F80, nan, 0x4000],
                  [0x8000, 0x0000, 0x8000, 0x0000]], dtype=np.uint16)
    keep = O.select_keep(g, 2, 4)
    assert keep.tolist() == [[True, True, False, False],
                             [True, True, False, False],
                             [True, False, True, False],
                             [True, True, False, False]]


# ------------------------------------------------------------- page figures ---

def test_page_configuration_counts(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))
    for (n, m), key in [((2, 4), "configs_2of4"), ((8, 16), "configs_8of16")]:
        subsets = list(combinations(range(m), n))
        x = np.full((len(subsets), m), 0x3F80, dtype=np.uint16)        # magnitude 1
        for r, s in enumerate(subsets):
            x[r, list(s)] = 0x4000                                       # magnitude 2
        keep = O.select_keep(x, n, m)
        masks = {tuple(np.flatnonzero(row)) for row in keep}
        assert masks == set(subsets)                                      # every mask reachable
        assert len(masks) == fig[key]["value"] == math.comb(m, n)


def test_page_slide_figures(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))
    ns = 4
    assert ns - 1 == fig["slide_6of8_windows"]["value"]
    assert O.lowered_k(8, ns) / 8 == fig["slide_6of8_gamma"]["value"]
    k = 4096
    executed = O.lowered_k(k, ns) // 2          # 2:4 hardware executes half of K'
    assert k / executed == pytest.approx(fig["slide_6of8_speedup"]["value"], rel=1e-15)
    assert 1 - 6 / 8 == fig["prune_frac_6of8"]["value"]
    assert 1 - 4 / 6 == pytest.approx(fig["prune_frac_4of6"]["value"])


# --------------------------------------------------------- hand-worked fixtures ---

def test_select_handworked(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "select_handworked.json")))["cases"]
    for c in cases:
        n, m = c["n"], c["m"]
        x = arr(c["x"])
        s, keep = O.sparsify(x, n, m)
        assert s.tolist() == arr(c["s"]).tolist()
        v, i = O.compress(x, n, m)
        assert v.tolist() == arr(c["values"]).tolist()
        assert i.tolist() == c["idx"]
        assert O.pack_mask(keep).tolist() == c["mask"]
        if "meta2bit" in c:
            assert O.pack_meta_2bit(i).tolist() == c["meta2bit"]


def test_slide_handworked(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "slide_handworked.json")))
    ns = fx["ns"]
    for c in fx["cases"]:
        wins = O.slide_windows(c["kept"], ns)
        assert wins == c["windows"]
        slots = [[p - 2 * w for p in pl] for w, pl in enumerate(wins)]
        assert slots == c["slots"]
        # through slide_lower on a one-group row with distinct values
        vals = np.array([[0x3F80 + 0x80 * j for j in range(6)]], dtype=np.uint16)
        idx = np.array([c["kept"]], dtype=np.uint8)
        vp, ip = O.slide_lower(vals, idx, 8, ns)
        assert ip.reshape(-1).tolist() == [s for sl in c["slots"] for s in sl]
        order = {p: j for j, p in enumerate(c["kept"])}
        assert vp.reshape(-1).tolist() == [int(vals[0, order[p]]) for pl in c["windows"] for p in pl]


# ------------------------------------------------------------------ invariants ---

@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32), (1, 4), (3, 8), (5, 16), (31, 32)])
def test_invariants(n, m):
    rng = np.random.default_rng(n * 100 + m)
    x = synth.student_t_bf16(rng, (7, m * 6), 4.0, 1.0)
    x[0, :m] = 0x8000                                  # -0 group
    x[1, :m] = 0x3F80                                  # all ties
    s, keep = O.sparsify(x, n, m)
    assert (keep.reshape(7, -1, m).sum(-1) == n).all()          # exactly n per group
    v, i = O.compress(x, n, m)
    assert (np.diff(i.reshape(7, -1, n).astype(int), axis=-1) > 0).all()   # ascending
    assert (i < m).all()
    assert (O.decompress(v, i, n, m, x.shape[1]) == s).all()     # round trip = S(X)
    # mask <-> idx bijection
    g = np.arange(x.shape[1] // m)
    pos = (g[None, :, None] * m + i.reshape(7, -1, n).astype(int)).reshape(7, -1)
    rebuilt = np.zeros_like(keep)
    np.put_along_axis(rebuilt, pos, True, axis=1)
    assert (rebuilt == keep).all()
    words = O.pack_mask(keep)
    pop = sum(bin(int(w)).count("1") for w in words.reshape(-1))
    assert pop == keep.sum()
    # values are x at idx
    assert (np.take_along_axis(x, pos, 1) == v).all()
    # compress(decompress(v, i)) == (v, i) when no kept value is +-0
    nz = (v & 0x7FFF) != 0
    rows = np.flatnonzero(nz.all(1))
    if len(rows):
        v2, i2 = O.compress(O.decompress(v[rows], i[rows], n, m, x.shape[1]), n, m)
        assert (v2 == v[rows]).all() and (i2 == i[rows]).all()


def test_n_equals_m_is_identity_and_dense_gemm():
    rng = np.random.default_rng(3)
    x = synth.normal_bf16(rng, (5, 64))
    w = synth.normal_bf16(rng, (9, 64), 0.02)
    for m in (4, 8, 16, 32):
        s, keep = O.sparsify(x, m, m)
        assert keep.all() and (s == x).all()
        assert (O.spmm_act(x, w, m, m) == O.gemm(x, w)).all()


def test_meta_2bit_roundtrip():
    rng = np.random.default_rng(4)
    x = synth.normal_bf16(rng, (6, 4 * 9))
    v, i = O.compress(x, 2, 4)
    meta = O.pack_meta_2bit(i)
    assert meta.shape == (6, (i.shape[1] + 3) // 4)
    assert (O.unpack_meta_2bit(meta, i.shape[1]) == i).all()


# ------------------------------------------------------------------ GEMM exactness ---

def gamma_f32(k):
    """gamma_K = K u / (1 - K u), u = 2^-24: the classical bound on the error of a K-term
    fp32 recursive sum of exact products, relative to the sum of their magnitudes."""
    u = Fraction(1, 2 ** 24)
    return k * u / (1 - k * u)


def assert_f32_sum_close(y, a_vals, b_vals):
    """y (an fp32-accumulated product of a [T][K] and b [O][K], exact products) is within
    gamma_K * (|a| |b|^T) of the exact product (computed in fp64, whose own error is far
    below that bound for these sizes)."""
    a = np.asarray(a_vals, np.float64)
    b = np.asarray(b_vals, np.float64)
    exact = a @ b.T
    bound = float(gamma_f32(a.shape[1])) * (np.abs(a) @ np.abs(b).T)
    assert (np.abs(np.asarray(y, np.float64) - exact) <= bound * 1.0001 + 1e-300).all()


def test_gemm_against_exact_rationals():
    """The fp32-accumulated product lies within gamma_K * sum|a b| of the exact rational
    result, and is not the exact result in general (the sums really round in fp32)."""
    rng = np.random.default_rng(5)
    a = synth.student_t_bf16(rng, (3, 48), 4.0, 1.0)
    b = synth.normal_bf16(rng, (4, 48), 0.02)
    y = O.gemm(a, b)
    inexact = 0
    for t in range(3):
        for o in range(4):
            exact = sum(Fraction(value_of(a[t, k])) * Fraction(value_of(b[o, k])) for k in range(48))
            absum = sum(abs(Fraction(value_of(a[t, k])) * Fraction(value_of(b[o, k]))) for k in range(48))
            assert abs(Fraction(y[t, o]) - exact) <= gamma_f32(48) * absum
            assert y[t, o] == f32_round(float(y[t, o]))          # an fp32 value
            inexact += Fraction(y[t, o]) != exact
    assert inexact > 0


def test_gemm_fp32_accumulation_order():
    """Closed forms that only an fp32 accumulator running over ascending k produces.
    a = [1, 2^-24, 2^-24]: each 2^-24 lands exactly half an ulp above 1 and rounds to even,
    so the result is 1 (fp64 gives 1 + 2^-23).  Reversed, the two small terms meet first
    and 1 + 2^-23 is exact.  A single term keeps its sign; no terms give +0."""
    one, tiny, mone = 0x3F80, 0x3380, 0xBF80          # 1, 2^-24, -1 in bf16
    b = np.array([[one, one, one]], dtype=np.uint16)
    assert O.gemm(np.array([[one, tiny, tiny]], np.uint16), b)[0, 0] == 1.0
    assert O.gemm(np.array([[tiny, tiny, one]], np.uint16), b)[0, 0] == 1.0 + 2.0 ** -23
    assert O.gemm_f64(np.array([[one, tiny, tiny]], np.uint16), b)[0, 0] == 1.0 + 2.0 ** -23
    # cancellation order: (1 + 2^-24) - 1 = 0 in fp32, 1 - 1 + 2^-24 = 2^-24
    assert O.gemm(np.array([[one, tiny, mone]], np.uint16), b)[0, 0] == 0.0
    assert O.gemm(np.array([[one, mone, tiny]], np.uint16), b)[0, 0] == 2.0 ** -24
    z = O.gemm(np.zeros((2, 0), np.uint16), np.zeros((3, 0), np.uint16))
    assert z.shape == (2, 3) and (z == 0).all() and not np.signbit(z).any()


def test_gemm_is_the_sequential_fp32_sum():
    """Brute force in pure Python: exact products (Python floats) rounded to fp32 through
    the C float conversion after every addition, k ascending."""
    rng = np.random.default_rng(25)
    a = synth.student_t_bf16(rng, (4, 40), 4.0, 1.0)
    b = synth.normal_bf16(rng, (5, 40), 0.02)
    y = O.gemm(a, b)
    for t in range(4):
        for o in range(5):
            acc = 0.0
            for k in range(40):
                acc = f32_round(acc + value_of(a[t, k]) * value_of(b[o, k]))
            assert y[t, o] == acc


def test_spmm_act_matches_masked_rational_product():
    rng = np.random.default_rng(6)
    x = synth.student_t_bf16(rng, (2, 32), 4.0, 0.5)
    w = synth.normal_bf16(rng, (3, 32), 0.02)
    y = O.spmm_act(x, w, 8, 16)
    for t in range(2):
        xv = [value_of(b) for b in x[t]]
        keep = brute_keep(xv[:16], 8) + brute_keep(xv[16:], 8)
        for o in range(3):
            exact = sum(Fraction(xv[k]) * Fraction(value_of(w[o, k])) for k in range(32) if keep[k])
            absum = sum(abs(Fraction(xv[k]) * Fraction(value_of(w[o, k]))) for k in range(32) if keep[k])
            assert abs(Fraction(y[t, o]) - exact) <= gamma_f32(32) * absum


# ------------------------------------------------------------------------- slide ---

@pytest.mark.parametrize("ns", [2, 3, 4, 5, 6])
def test_slide_exhaustive_masks(ns):
    m = 2 * ns
    n = 2 * ns - 2
    count = 0
    for kept in combinations(range(m), n):
        wins = O.slide_windows(list(kept), ns)
        assert all(len(w) == 2 for w in wins)
        for w, pl in enumerate(wins):
            assert all(2 * w <= p <= 2 * w + 3 for p in pl)
        assert sorted(p for pl in wins for p in pl) == list(kept)
        count += 1
    assert count == math.comb(m, n)
    # N-2 windows hold at most 2N-4 < 2N-2 values: never enough
    assert 2 * (ns - 2) < n
    assert O.lowered_k(m, ns) == 4 * (ns - 1)


def test_slide_pipeline_reconstructs_and_multiplies():
    rng = np.random.default_rng(7)
    ns = 4
    w = synth.normal_bf16(rng, (6, 64), 0.02)
    w[0, :8] = 0x3F80                                  # fully tied group
    x = synth.normal_bf16(rng, (5, 64))
    v, i = O.compress(w, 6, 8)
    vp, ip = O.slide_lower(v, i, 64, ns)
    assert vp.shape == (6, O.lowered_k(64, ns) // 2)
    pruned, _ = O.sparsify(w, 6, 8)
    assert (O.slide_scatter_back(vp, ip, 64, ns) == pruned).all()
    y_slide = O.spmm_slide(x, vp, ip, ns)
    xl = O.lift(x, ns)
    for t in range(5):
        for o in range(6):
            wd = O.decompress(vp[o:o + 1], ip[o:o + 1], 2, 4, O.lowered_k(64, ns))[0]
            exact_lifted = sum(Fraction(value_of(xl[t, k])) * Fraction(value_of(wd[k])) for k in range(len(wd)))
            exact_dense = sum(Fraction(value_of(x[t, k])) * Fraction(value_of(pruned[o, k])) for k in range(64))
            assert exact_lifted == exact_dense
            absum = sum(abs(Fraction(value_of(xl[t, k])) * Fraction(value_of(wd[k]))) for k in range(len(wd)))
            assert abs(Fraction(y_slide[t, o]) - exact_dense) <= gamma_f32(len(wd)) * absum


def test_lift_positions():
    x = np.arange(16, dtype=np.uint16)[None, :]
    xl = O.lift(x, 4)
    assert xl[0].tolist() == [0, 1, 2, 3, 2, 3, 4, 5, 4, 5, 6, 7, 8, 9, 10, 11, 10, 11, 12, 13, 12, 13, 14, 15]


# ------------------------------------------------------------------------ hybrid ---

def test_hybrid_column_choice_constructed():
    rng = np.random.default_rng(8)
    o, k, kd = 16, 32, 8
    w = synth.normal_bf16(rng, (o, k), 0.02)
    big = [3, 5, 17, 18, 20, 26, 30, 31]
    for c in big:
        w[:, c] = synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(w[:, c]) * np.float32(64.0))
    sp, de = O.hybrid_columns(w, kd)
    assert de.tolist() == big
    assert sp.tolist() == [c for c in range(k) if c not in big]
    # norm ties resolve to the lower column
    w2 = np.full((4, 8), 0x3F80, dtype=np.uint16)
    sp2, de2 = O.hybrid_columns(w2, 3)
    assert de2.tolist() == [0, 1, 2]


def test_hybrid_norms_exact():
    rng = np.random.default_rng(9)
    w = synth.normal_bf16(rng, (40, 6), 0.02)
    c = O.column_sq_norms(w)
    for j in range(6):
        exact = sum(Fraction(value_of(w[o, j])) ** 2 for o in range(40))
        assert abs(Fraction(c[j]) - exact) <= exact * Fraction(2.0 ** -50)


@pytest.mark.parametrize("kd", [0, 8, 32])
def test_hybrid_split_sum(kd):
    rng = np.random.default_rng(10 + kd)
    o, k = 12, 32
    w = synth.normal_bf16(rng, (o, k), 0.02)
    x = synth.normal_bf16(rng, (5, k))
    sp, de, v, i, wd = O.hybrid_pack(w, kd)
    assert len(sp) + len(de) == k and len(de) == kd
    y = O.hybrid_gemm(x, sp, de, v, i, wd)
    # W_h: sparse columns replaced by their 2:4 pruned values scattered back
    wh = w.copy()
    if len(sp):
        ws_pruned = O.decompress(v, i, 2, 4, len(sp))
        wh[:, sp] = ws_pruned
        # the sparse region is exactly the 2:4 magnitude pruning of the permuted columns
        assert (ws_pruned == O.sparsify(np.ascontiguousarray(w[:, sp]), 2, 4)[0]).all()
    assert_f32_sum_close(y, O.bf16_to_f64(x), O.bf16_to_f64(wh))
    if kd == k:
        # all columns dense, in ascending order: exactly the plain product
        assert (de == np.arange(k)).all() and (y == O.gemm(x, w)).all()
    if kd == 0:
        assert (sp == np.arange(k)).all()
        assert (y == O.gemm(x, O.sparsify(w, 2, 4)[0])).all()


# --------------------------------------------------------------------------- fp8 ---

def test_fp8_decode_all_codes_vs_torch():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2
    assert (ours[~nan] == ref[~nan]).all()
    assert np.nanmax(ours) == 448.0
    # every finite code is exactly representable in bf16
    b = synth.bf16_bits_from_f32(ours[~nan].astype(np.float32))
    assert (synth.f32_from_bf16_bits(b).astype(np.float64) == ours[~nan]).all()


def test_fp8_layer_equals_scaled_bf16_layer():
    rng = np.random.default_rng(14)
    w = synth.normal_bf16(rng, (6, 64), 0.02)
    x = synth.student_t_bf16(rng, (4, 64), 4.0, 1.0)
    q, s = synth.fp8_e4m3_quantize_rows(w)
    y8 = O.spmm_act_fp8(x, q, s, 8, 16)
    wdeq = O.fp8_e4m3_to_f64(q) * s[:, None].astype(np.float64)
    sx, _ = O.sparsify(x, 8, 16)
    exact = O.bf16_to_f64(sx) @ wdeq.T
    bound = float(gamma_f32(64)) * (np.abs(O.bf16_to_f64(sx)) @ np.abs(wdeq).T) + 2.0 ** -24 * np.abs(exact)
    assert (np.abs(y8 - exact) <= bound * 1.0001 + 1e-30).all()


# ----------------------------------------------------------- scored selection ---

def f32_round(v):
    """Round a Python float (fp64, here always the exact product) to fp32, ties to even,
    subnormals kept: the C conversion behind struct, independent of numpy."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


@pytest.mark.parametrize("m", [4, 8, 16, 32])
def test_scored_unit_scale_is_act(m):
    """c = 1 for every column: |x| * 1 is |x| exactly, so the weighted score ranks like
    the ACT magnitude (ties included) and the masks agree."""
    rng = np.random.default_rng(m)
    x = rng.choice(np.array(ALPHABET + [0x3E80, 0x4100], dtype=np.uint16), size=(40, 4 * m))
    x[:20] = synth.student_t_bf16(rng, (20, 4 * m), 4.0, 0.5)
    ones = np.ones(4 * m, np.float32)
    for n in sorted({1, m // 4 or 1, m // 2, m - 1, m}):
        assert (O.select_keep_scored(x, ones, n, m, O.SCORE_ACT_WEIGHTED) == O.select_keep(x, n, m)).all()
    # any power-of-two scale common to all columns ranks the same way
    assert (O.select_keep_scored(x, ones * 0.125, m // 2, m, O.SCORE_ACT_WEIGHTED)
            == O.select_keep(x, m // 2, m)).all()


@pytest.mark.parametrize("m,n", [(4, 2), (8, 3), (8, 4), (16, 8)])
def test_scored_bruteforce_rounded_products(m, n):
    """Each score is the exact product |x| * c (exact in fp64 for bf16 x fp32) rounded
    once to fp32; the kept set is the first n-subset of largest score sum (brute force).
    Tiny values put some products in the fp32 subnormal range; repeated column scales
    and repeated |x| force ties, which rounding can also create."""
    rng = np.random.default_rng(100 * m + n)
    rows = 24
    x = synth.student_t_bf16(rng, (rows, 2 * m), 4.0, 0.5)
    x[3] = x[3, 0]                                        # one row of equal magnitudes
    x[4, :m] = 0x0080                                     # bf16 min normal (2^-126)
    x[5] = rng.choice(np.array([0x3F80, 0xBF80, 0x3F81, 0x3F7F], dtype=np.uint16), size=2 * m)
    c = rng.uniform(0.25, 4.0, size=2 * m).astype(np.float32)
    c[1::3] = c[0]                                        # repeated scales
    c[m // 2] = np.float32(2.0 ** -20)                    # products below the normal range
    c[m - 1] = np.float32(1.0 + 2.0 ** -23)               # rounding-sensitive scale
    keep = O.select_keep_scored(x, c, n, m, O.SCORE_ACT_WEIGHTED)
    if m >= 16:
        rows = 8
    for r in range(rows):
        for g in range(2):
            scores = [f32_round(abs(value_of(x[r, g * m + i])) * float(c[g * m + i])) for i in range(m)]
            assert list(keep[r, g * m:(g + 1) * m]) == brute_keep(scores, n), (r, g)


def test_scored_weight_mode_ignores_x():
    """WT: the score is the column's weight magnitude alone, so every row keeps the same
    positions: per group the n largest c_k, ties to the lower index (brute force)."""
    rng = np.random.default_rng(7)
    m, n = 16, 8
    x = synth.student_t_bf16(rng, (9, 3 * m), 4.0, 0.5)
    c = rng.choice(np.array([0.5, 1.0, 1.5, 3.0], np.float32), size=3 * m)
    keep = O.select_keep_scored(x, c, n, m, O.SCORE_WEIGHT)
    for g in range(3):
        ref = brute_keep([float(v) for v in c[g * m:(g + 1) * m]], n)
        for r in range(x.shape[0]):
            assert list(keep[r, g * m:(g + 1) * m]) == ref


@pytest.mark.parametrize("mode", [0, 1])
def test_scored_invariants(mode):
    """Exactly n kept per group; every kept score beats every pruned one under (score
    descending, index ascending); S(X) copies kept bits and zeroes the rest."""
    rng = np.random.default_rng(11 + mode)
    m, n = 16, 8
    x = synth.student_t_bf16(rng, (50, 8 * m), 4.0, 0.5)
    c = (np.abs(rng.standard_normal(8 * m)) + 0.01).astype(np.float32)
    y, keep = O.sparsify_scored(x, c, n, m, mode)
    s = O.selection_scores(x, c, mode)
    assert (keep.reshape(50, 8, m).sum(-1) == n).all()
    for r in range(50):
        for g in range(8):
            sl = slice(g * m, (g + 1) * m)
            kept = [i for i in range(m) if keep[r, sl][i]]
            pruned = [i for i in range(m) if not keep[r, sl][i]]
            for i in kept:
                for j in pruned:
                    assert (s[r, sl][i] > s[r, sl][j]) or (s[r, sl][i] == s[r, sl][j] and i < j)
    assert (y[keep] == x[keep]).all() and (y[~keep] == 0).all()


def test_scored_rounding_makes_ties():
    """The score is one rounded fp32 product: 1 * (1 + 2^-7 + 2^-23) and
    (1 + 2^-7) * (1 + 2^-23) differ by 2^-30 exactly but are the same fp32 number, so
    with n = 1 the lower index wins (an exact-arithmetic score would keep index 1)."""
    x = np.array([[0x3F80, 0x3F81, 0x3F00, 0x3F00]], np.uint16)          # 1, 1 + 2^-7, .5, .5
    c = np.array([1 + 2.0 ** -7 + 2.0 ** -23, 1 + 2.0 ** -23, 1.0, 1.0], np.float32)
    assert float(c[0]) == 1 + 2.0 ** -7 + 2.0 ** -23 and float(c[1]) == 1 + 2.0 ** -23
    exact = [abs(value_of(x[0, i])) * float(c[i]) for i in range(4)]
    assert exact[1] > exact[0] and f32_round(exact[1]) == f32_round(exact[0])
    assert list(O.select_keep_scored(x, c, 1, 4, O.SCORE_ACT_WEIGHTED)[0]) == [True, False, False, False]


# ------------------------------------------------------------------ Spense GLU ---

def test_spense_scores_exact_small_integers():
    """Integer-valued weights and Hessian roots keep every sum exact in fp64, so the
    scores equal the rational formula: sum_j |Wg_ij| h_j + sum_j |Wu_ij| h_j + m_i sum_o |Wd_oi|."""
    rng = np.random.default_rng(3)
    i_n, h = 12, 8
    ints = np.array([-3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
    wg = arr(rng.choice(ints, (i_n, h)).tolist())
    wu = arr(rng.choice(ints, (i_n, h)).tolist())
    wd = arr(rng.choice(ints, (h, i_n)).tolist())
    hs_in = rng.choice([0.5, 1.0, 2.0, 3.0], h)
    hs_mid = rng.choice([0.25, 1.0, 5.0], i_n)
    got = O.spense_glu_scores(wg, wu, wd, hs_in, hs_mid)
    for i in range(i_n):
        ref = sum(abs(Fraction(value_of(wg[i, j]))) * Fraction(hs_in[j]) for j in range(h))
        ref += sum(abs(Fraction(value_of(wu[i, j]))) * Fraction(hs_in[j]) for j in range(h))
        ref += Fraction(hs_mid[i]) * sum(abs(Fraction(value_of(wd[o, i]))) for o in range(h))
        assert Fraction(got[i]) == ref


def test_spense_scores_fixed_order():
    """The sums run left to right in fp64: 1 + 2^-53 + 2^-53 gives 1 (each small term is
    lost to round-to-even), where an exact or pairwise sum would give 1 + 2^-52."""
    tiny = 2.0 ** -53
    wg = arr([[1.0, tiny, tiny]])
    zero = arr([[0.0, 0.0, 0.0]])
    got = O.spense_glu_scores(wg, zero, arr([[0.0], [0.0], [0.0]]), np.ones(3), np.ones(1))
    assert got[0] == 1.0 and 1.0 + 2 * tiny != 1.0


def test_spense_order_ties_and_layout():
    scores = np.array([2.0, 5.0, 5.0, 1.0, 5.0, 0.0])
    perm = O.spense_order(scores, 2)
    # dense: the two largest, 5.0 at indices 1 and 2 (index 4 loses the tie); sparse first
    assert list(perm) == [0, 3, 4, 5, 1, 2]
    assert list(O.spense_order(scores, 0)) == list(range(6))
    assert sorted(O.spense_order(scores, 6)) == list(range(6)) and list(O.spense_order(scores, 6)) == list(range(6))
    assert list(O.spense_order_tail(6, 2)) == list(range(6))


def _silu(v):
    return v / (1.0 + np.exp(-v))


def test_spense_glu_permutation_invariance():
    """A GLU MLP gives the same output when gate/up rows and down columns are permuted
    together.  Spense MLP = down input-split over silu(gate) * up, each from the output-
    split products in permuted order; it equals the plain MLP on the weights with the
    same 2:4 pruning applied to the sparse rows of gate/up and sparse columns of down."""
    rng = np.random.default_rng(21)
    t, h, i_n, n_dense = 5, 32, 48, 12
    x = synth.normal_bf16(rng, (t, h))
    wg = synth.normal_bf16(rng, (i_n, h), 0.02)
    wu = synth.normal_bf16(rng, (i_n, h), 0.02)
    wd = synth.normal_bf16(rng, (h, i_n), 0.02)
    scores = O.spense_glu_scores(wg, wu, wd, np.abs(rng.standard_normal(h)), np.abs(rng.standard_normal(i_n)))
    perm = O.spense_order(scores, n_dense)
    ns = i_n - n_dense
    gv, gi, gd = O.spense_pack(wg, perm, ns, 0)
    uv, ui, ud = O.spense_pack(wu, perm, ns, 0)
    dv, di, dd = O.spense_pack(wd, perm, ns, 1)
    a = _silu(O.outsplit_gemm(x, gv, gi, gd, h)) * O.outsplit_gemm(x, uv, ui, ud, h)   # permuted order
    y = a[:, :ns] @ O.bf16_to_f64(O.decompress(dv, di, 2, 4, ns)).T + a[:, ns:] @ O.bf16_to_f64(dd).T
    # plain MLP on the equivalently pruned weights, original index order
    wg_e, wu_e, wd_e = wg.copy(), wu.copy(), wd.copy()
    sp = perm[:ns]
    wg_e[sp] = O.sparsify(wg[sp], 2, 4)[0]
    wu_e[sp] = O.sparsify(wu[sp], 2, 4)[0]
    wd_e[:, sp] = O.sparsify(np.ascontiguousarray(wd[:, sp]), 2, 4)[0]
    xf = O.bf16_to_f64(x)
    ref = (_silu(xf @ O.bf16_to_f64(wg_e).T) * (xf @ O.bf16_to_f64(wu_e).T)) @ O.bf16_to_f64(wd_e).T
    # gate / up are fp32-accumulated (relative error ~1e-7 of their sums)
    assert np.allclose(y, ref, rtol=1e-5, atol=1e-9)
    # a permutation that does not keep gate/up rows and down columns together changes it
    bad = O.bf16_to_f64(O.decompress(dv, di, 2, 4, ns))[:, ::-1]
    y_bad = a[:, :ns] @ bad.T + a[:, ns:] @ O.bf16_to_f64(dd).T
    assert not np.allclose(y_bad, ref, rtol=1e-3)


@pytest.mark.parametrize("axis", [0, 1])
def test_spense_pack_regions(axis):
    rng = np.random.default_rng(5 + axis)
    w = synth.normal_bf16(rng, (24, 40), 0.02)
    n = w.shape[axis]
    perm = rng.permutation(n).astype(np.int32)
    ns = 16
    v, i, wd = O.spense_pack(w, perm, ns, axis)
    ws = w[perm[:ns]] if axis == 0 else np.ascontiguousarray(w[:, perm[:ns]])
    kk = ws.shape[1]
    assert (O.decompress(v, i, 2, 4, kk) == O.sparsify(ws, 2, 4)[0]).all()
    assert (wd == (w[perm[ns:]] if axis == 0 else w[:, perm[ns:]])).all()


# ------------------------------------------------------------- fp8 activations ---

def test_e4m3_encode_against_torch():
    """The encoder written from the format definition agrees with torch's fp32 ->
    float8_e4m3fn conversion: every finite code value, every midpoint between neighbouring
    codes (ties to even), and random values across the normal and subnormal ranges."""
    import torch

    codes = np.array([c for c in range(256) if not np.isnan(O.fp8_e4m3_to_f64(np.uint8(c)))], np.uint8)
    vals = O.fp8_e4m3_to_f64(codes)
    assert (O.e4m3_encode(vals) == codes).all()
    pos = np.sort(np.unique(np.abs(vals)))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(8)
    rnd = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-2 ** -6, 2 ** -6, 2000),
                          rng.uniform(-1, 1, 2000) * 2.0 ** -10])
    for v in (np.concatenate([mids, -mids]), rnd):
        v32 = v.astype(np.float32)
        ref = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (O.e4m3_encode(v32.astype(np.float64)) == ref).all()


def test_quantize_tokens_properties():
    """Each row's largest magnitude maps to +-448 exactly; every value is reproduced by
    dec(q) * s within half an e4m3 step (relative 2^-4 in the normal range, 2^-10 s below
    it); the scale is amax / 448 in fp32; an all-zero row gets scale 1 and zero codes."""
    rng = np.random.default_rng(9)
    x = synth.student_t_bf16(rng, (40, 512), 4.0, 0.5)
    x[7] = 0
    q, s = O.quantize_tokens(x)
    xf = O.bf16_to_f64(x)
    amax = np.abs(xf).max(1)
    for t in range(40):
        if amax[t] == 0:
            assert s[t] == 1.0 and (q[t] == 0).all()
            continue
        assert s[t] == np.float32(np.float32(amax[t]) / np.float32(448.0))
        j = int(np.argmax(np.abs(xf[t])))
        assert q[t, j] in (0x7E, 0xFE)
        d = O.fp8_e4m3_to_f64(q[t]) * float(s[t])
        err = np.abs(d - xf[t])
        small = np.abs(xf[t]) < 2.0 ** -6 * float(s[t])
        assert (err[~small] <= 2.0 ** -4 * np.abs(xf[t][~small]) * (1 + 1e-6)).all()
        assert (err[small] <= 2.0 ** -10 * float(s[t]) * (1 + 1e-6)).all()


@pytest.mark.parametrize("ns", [2, 4])
def test_w8a8_slide_is_the_dequantized_dense_product(ns):
    """Lifting X and lowering W preserve the product, so the fp8 result must equal the
    dense product of the dequantized tokens with the weight codes scattered back to their
    original positions -- a route that never lifts."""
    rng = np.random.default_rng(10 + ns)
    t, o, k = 9, 12, 64
    x = synth.student_t_bf16(rng, (t, k), 4.0, 0.5)
    w = synth.normal_bf16(rng, (o, k), 0.02)
    if ns == 2:
        vals, idx = O.compress(w, 2, 4)
        w8, ws = synth.fp8_e4m3_quantize_rows(vals)
        wd = O.decompress(w8.astype(np.uint16), idx, 2, 4, k).astype(np.uint8)
    else:
        v, i = O.compress(w, 6, 8)
        vp, ip = O.slide_lower(v, i, k, ns)
        w8, ws = synth.fp8_e4m3_quantize_rows(vp)
        idx = ip
        wd = O.slide_scatter_back(w8.astype(np.uint16), ip, k, ns).astype(np.uint8)
    got = O.spmm_w8a8_slide(x, w8, idx, ws, k, ns)
    q, st = O.quantize_tokens(x)
    xa = O.fp8_e4m3_to_f64(q) * st[:, None].astype(np.float64)
    wa = O.fp8_e4m3_to_f64(wd) * ws[:, None].astype(np.float64)
    ref = xa @ wa.T
    # fp32 accumulation over the lifted length, then two scale roundings
    kp = O.lowered_k(k, ns) if ns > 2 else k
    bound = float(gamma_f32(kp)) * (np.abs(xa) @ np.abs(wa).T) + 2 * 2.0 ** -24 * np.abs(ref) * 1.0001
    assert (np.abs(got - ref) <= bound + 1e-30).all()


# ------------------------------------------------- error mitigation: PTS and VAR ---

def bf16_round_py(v):
    """Pure-Python bf16 rounding of a Python float: to fp32 through the C conversion, then
    round-to-nearest-even on the bit pattern (independent of the oracle's helpers)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u & 0xFFFF


def test_pts_mean_exact_rows_and_order_free():
    """mu is the row mean: exactly, where the mean is an fp32 value; within one fp32
    rounding plus 2^-37 max|x| of the exact rational mean otherwise -- also across a 2^200
    dynamic range; and bit-identical under any permutation of the row."""
    x = arr([[1, 2, 3, 4, 5, 6, 7, 8], [-3, -1, 0.5, 0.5, 2, 0, 0, 1], [0, 0, 0, 0, 0, 0, 0, 0],
             ["-0", 0, "-0", 0, 0, 0, 0, 0]])
    mu = O.pts_row_mean(x)
    assert mu.tolist() == [4.5, 0.0, 0.0, 0.0] and not np.signbit(mu[2:]).any()
    rng = np.random.default_rng(31)
    xs = synth.student_t_bf16(rng, (6, 160), 4.0, 0.5)
    xs[5, 3] = bits_of(2.0 ** 100)
    xs[5, 7] = bits_of(-(2.0 ** -100))
    xs[5, 9] = 0x0001                                     # a subnormal
    mu = O.pts_row_mean(xs)
    for r in range(6):
        vals = [Fraction(value_of(b)) for b in xs[r]]
        exact = sum(vals) / len(vals)
        big = max(abs(v) for v in vals)
        assert abs(Fraction(float(mu[r])) - exact) <= abs(exact) * Fraction(1, 2 ** 24) + big / 2 ** 37
        for _ in range(3):
            perm = rng.permutation(160)
            assert O.pts_row_mean(xs[r:r + 1, perm])[0].view(np.uint32) == mu[r].view(np.uint32)
    with pytest.raises(ValueError):
        O.pts_row_mean(arr([[1, 2, 3, float("inf")]]))


def test_pts_zero_static_shift_is_act():
    """A static shift of zero leaves every value (and -0) unchanged: S-PTS reduces to ACT."""
    rng = np.random.default_rng(32)
    x = synth.student_t_bf16(rng, (5, 64), 4.0, 0.5)
    x[0, :4] = 0x8000
    for n, m in ((2, 4), (8, 16), (16, 32)):
        s, keep, mu, alpha = O.sparsify_pts(x, n, m, O.PTS_STATIC, np.zeros(64, np.float32))
        s_act, keep_act = O.sparsify(x, n, m)
        assert mu is None and alpha is None
        assert (keep == keep_act).all()
        # x - 0 rounds -0 to +0 in fp32 (RNE); kept values are otherwise identical
        assert (s[s_act != 0x8000] == s_act[s_act != 0x8000]).all()


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8)])
def test_pts_shift_then_select_bruteforce(n, m):
    """Tiny rows: the shift computed from the exact rational mean, rounded to fp32 and then
    bf16 in pure Python, and the kept set chosen by brute force over all n-subsets."""
    rng = np.random.default_rng(33 + m)
    for trial in range(40):
        k = m * int(rng.integers(1, 4))
        x = synth.student_t_bf16(rng, (1, k), 4.0, 0.5)
        if trial % 4 == 0:                                 # many ties after the shift
            x[0] = np.array([bits_of(v) for v in rng.choice([0.5, 1.0, 1.5, 2.0, -1.0], size=k)], np.uint16)
        vals = [Fraction(value_of(b)) for b in x[0]]
        mean = sum(vals) / k
        mu = struct.unpack("<f", struct.pack("<f", float(mean)))[0]     # exact mean, one rounding
        s, keep, mu_o, _ = O.sparsify_pts(x, n, m, O.PTS_DYNAMIC)
        assert mu_o[0] == mu
        shifted = [bf16_round_py(float(Fraction(value_of(b)) - Fraction(mu))) for b in x[0]]
        # fp32(x - mu) is one rounding of the exact difference; bf16 rounds that result
        sh32 = [f32_round(value_of(b) - mu) for b in x[0]]
        assert shifted == [bf16_round_py(v) for v in sh32]
        for g in range(k // m):
            grp = [value_of(b) for b in shifted[g * m:(g + 1) * m]]
            bk = brute_keep(grp, n)
            assert list(keep[0, g * m:(g + 1) * m]) == bk
            for j in range(m):
                want = shifted[g * m + j] if bk[j] else 0
                assert int(s[0, g * m + j]) == want


def test_pts_rank_one_term_undoes_the_shift():
    """Without pruning (n = m) the shift must cancel exactly: on rows whose shifted values
    are exact in bf16, Y = (x - mu) W^T + mu (W 1) equals x W^T up to the fp32 rounding of
    the product (exact rational check).  With pruning, Y equals S(x~) W^T + mu (W 1)."""
    rng = np.random.default_rng(34)
    x = arr([[1, 2, 3, 4, 5, 6, 7, 8] * 2, [-3, 5, 1, 1, 2, 0, 4, 6] * 2])     # means 4.5, 2
    w = synth.normal_bf16(rng, (3, 16), 0.02)
    wv = O.bf16_to_f64(w)
    v = O.weight_sums(wv)
    for n in (8, 4):
        y, s, keep, mu, _ = O.spmm_pts(x, w, n, 8, O.PTS_DYNAMIC, col_shift=v)
        assert mu.tolist() == [4.5, 2.0]
        for t in range(2):
            for o in range(3):
                a = [Fraction(value_of(b)) for b in (x[t] if n == 8 else s[t])]
                if n == 8:
                    exact = sum(a[k] * Fraction(value_of(w[o, k])) for k in range(16))
                else:
                    exact = sum(a[k] * Fraction(value_of(w[o, k])) for k in range(16)) + \
                        Fraction(float(mu[t])) * Fraction(float(v[o]))
                absum = sum(abs(Fraction(value_of(b)) * Fraction(value_of(w[o, k])))
                            for k, b in enumerate(s[t])) + abs(Fraction(float(mu[t])) * Fraction(float(v[o])))
                # fp32 product, fp32 rounding of v, fp64 epilogue
                tol = gamma_f32(16) * absum + abs(Fraction(float(mu[t]))) * Fraction(1, 2 ** 24) * \
                    sum(abs(Fraction(value_of(w[o, k]))) for k in range(16)) + Fraction(1, 2 ** 40)
                assert abs(Fraction(y[t, o]) - exact) <= tol, (n, t, o)


def test_var_restores_the_row_variance():
    """alpha_t S(x~_t) has the variance of x~_t (up to alpha's fp32 rounding); a row whose
    pruned form has no variance gets alpha = 1."""
    rng = np.random.default_rng(35)
    x = synth.student_t_bf16(rng, (6, 256), 4.0, 0.5)
    x[5] = 0
    for mode in (O.PTS_VAR, O.PTS_VAR | O.PTS_DYNAMIC):
        s, keep, mu, alpha = O.sparsify_pts(x, 8, 16, mode)
        xs = O.pts_shift(x, shift_rows=mu) if mode & O.PTS_DYNAMIC else x
        for r in range(5):
            before = np.var(O.bf16_to_f64(xs[r]))
            after = np.var(float(alpha[r]) * O.bf16_to_f64(s[r]))
            assert abs(after - before) <= 3e-7 * before
            assert alpha[r] > 1.0                       # pruning half the entries shrinks the variance
        assert alpha[5] == 1.0


def test_weight_sums_against_exact_sums():
    rng = np.random.default_rng(36)
    w = synth.normal_bf16(rng, (5, 96), 0.02)
    c = rng.standard_normal(96).astype(np.float32)
    for shift in (None, c):
        v = O.weight_sums(O.bf16_to_f64(w), shift)
        for o in range(5):
            exact = sum(Fraction(value_of(w[o, k])) * (1 if shift is None else Fraction(float(c[k])))
                        for k in range(96))
            absum = sum(abs(Fraction(value_of(w[o, k])) * (1 if shift is None else Fraction(float(c[k]))))
                        for k in range(96))
            assert abs(Fraction(float(v[o])) - exact) <= abs(exact) / 2 ** 24 + absum * 96 / 2 ** 52
