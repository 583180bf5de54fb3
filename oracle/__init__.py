"""CPU oracle for the N:M structured-sparse linear layer Y = S(X) . W^T.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The library's GPU path never calls it, and
it shares no code, table or helper with the GPU path: it is written from the papers'
descriptions, plain and unblocked, so that a reader can check each step by eye.

Conventions
-----------
* bf16 tensors are numpy ``uint16`` arrays of bit patterns, row-major, K fastest.
* Matrix products follow the workloads' "fp32 accumulate": ``gemm`` and the products
  built on it run the plain single-threaded C loop of ``gemm_f32.c`` -- one fp32
  accumulator per output, products added in ascending k, every sum rounded to nearest
  even (bf16 x bf16 and bf16 x e4m3 products are exact in fp32).  ``gemm_f64`` is the
  library fp64 product of the same operands, used only for error bounds and whole-output
  projection checks, never as the parity reference.
* "Group" = m contiguous elements along K; group g of a row covers k in [g*m, g*m+m).

Sources (cited by page title and section)
-----------------------------------------
[FLEX]  "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity via
        Benchmarking Lightweight Post-Training Sparsification Approaches"
        - technical summary section 1 (configuration counts 6 and 12,870; metadata cost),
          section 2.A (ACT score = activation magnitude; WT and Amber-Pruner scores from
          weight magnitudes), section 2.C (patterns 2:4, 4:8,
          8:16, 16:32 along the reduction dimension).
[SLIDE] "SlideSparse: Fast and Flexible (2N-2):2N Structured Sparsity"
        - technical summary section 2.A (N-1 overlapping windows of width 4, stride 2,
          at most 2 non-zeros each, overflow carried to the next window; gamma=(2N-2)/N),
          section 2.B (activation lifting), section 2.C (offline packer), section 4
          (theoretical speedup N/(N-1)).
[SPENSE] "SpenseGPT: Practical One-shot Pruning Enabling Sparse and Dense GEMMs for LLM
        Inference" - technical summary section 2.A (dense region + 2:4 region, input
        split with accumulation), section 2.B (dense indices permuted into a contiguous
        block).

Readings where the pages are silent (each is listed in the design notes):
* Ties in the magnitude order go to the lower in-group index.
* Magnitude order = order of the 15 low bits of the bf16 pattern (sign dropped).  This
  equals the |x| order for every finite or infinite value; +0 and -0 tie; a NaN ranks
  above infinity.
* Pruned entries of S(X) are +0.0 (bits 0x0000); kept entries are copied bit for bit.
* Index metadata: one byte per kept value holding its in-group position (0..m-1), kept
  values stored in ascending position; for 2:4 the same positions can be packed two bits
  each (byte j//4, bits 2*(j%4)) where j is the kept-value slot.
* Sliding windows: kept positions are visited in ascending order and each goes to the
  lowest-numbered window that covers it and still holds fewer than two ("overflow moves
  to the next window").  Window w of group g occupies lowered positions
  g*4(N-1) + 4w + s holding original position g*2N + 2w + s.
* Hybrid split: dense columns = the K_d columns with the largest L2 norm over the output
  dimension (sum of squares in fp64, o ascending; ties to the lower column); sparse
  region first, then dense region, each in ascending original column order; the sparse
  region is pruned 2:4 by magnitude over consecutive permuted columns.
* fp8 weights: OCP E4M3FN codes with one fp32 scale per output row, applied after the
  K reduction.
* Per-token fp8 activations (quantize_tokens): symmetric absmax scaling, codes of
  x * fp32(448 / amax).  PARITY UNPINNED in that one choice: dividing by
  fp32(amax / 448) is an equally plain reading that differs by one code at rounding
  boundaries, and the pages give no scheme.  Its properties (every code within half an
  e4m3 step of x/s, the row maximum at +-448, zero rows, the encoder against an
  independent library) are pinned.
* Activation mitigations ([FLEX] 2.B): D-PTS shifts each token row by its mean before
  the selection, S-PTS by a given per-channel vector, and the shift is undone by the
  rank-one term mu_t * (W . 1)_o (or (W . c)_o); VAR scales each pruned row to its
  unpruned variance.  The page names these steps without formulas: these are the
  plainest readings, pinned by their reductions and identities (zero shift = ACT, the
  rank-one identity, the restored variance), not by printed values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

__all__ = [
    "magnitude_key", "bf16_to_f64", "select_keep", "sparsify", "pack_mask", "compress",
    "pack_meta_2bit", "unpack_meta_2bit", "decompress", "slide_windows",
    "slide_lower", "slide_scatter_back", "lift", "column_sq_norms", "hybrid_columns",
    "hybrid_pack", "gemm", "gemm_f64", "gemm_f32_values", "build_c", "spmm_act", "spmm_slide", "hybrid_gemm", "fp8_e4m3_to_f64",
    "spmm_act_fp8", "lowered_k", "SCORE_ACT_WEIGHTED", "SCORE_WEIGHT", "selection_scores",
    "select_keep_scored", "sparsify_scored", "spense_glu_scores", "spense_order", "spense_order_tail",
    "spense_pack", "outsplit_gemm", "e4m3_encode", "quantize_tokens", "f32_from_bf16", "spmm_w8a8_slide",
    "bf16_from_f32_rne", "pts_row_mean", "pts_shift", "sparsify_pts", "var_scale", "weight_sums", "spmm_pts",
    "PTS_DYNAMIC", "PTS_STATIC", "PTS_VAR",
]


# ----------------------------------------------------------------------------- bf16 ---

def magnitude_key(bits: np.ndarray) -> np.ndarray:
    """Magnitude order key of a bf16 bit pattern: the 15 bits below the sign.
    [FLEX] 2.A: the ACT score is the absolute value of the activation."""
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.int32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- select ---

def _groups(bits: np.ndarray, m: int) -> np.ndarray:
    r, k = bits.shape
    if k % m:
        raise ValueError("K must be a multiple of m")
    return bits.reshape(r, k // m, m)


def select_keep(bits: np.ndarray, n: int, m: int, row_chunk: int = 256) -> np.ndarray:
    """Boolean keep mask of the per-group magnitude top-n.  [FLEX] 2.A, 2.C.

    In every group of m contiguous values along K, position i has
        rank_i = #{j : key_j > key_i} + #{j < i : key_j == key_i}
    and is kept iff rank_i < n (largest magnitudes first, ties to the lower index).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    if not (1 <= n <= m):
        raise ValueError("need 1 <= n <= m")
    r, k = bits.shape
    keep = np.empty((r, k), dtype=bool)
    lower = np.tril(np.ones((m, m), dtype=bool), k=-1)   # lower[i, j] = (j < i)
    for r0 in range(0, r, row_chunk):
        key = magnitude_key(_groups(bits[r0:r0 + row_chunk], m))   # [R, G, m]
        ki = key[..., :, None]                                     # key_i
        kj = key[..., None, :]                                     # key_j
        rank = (kj > ki).sum(-1) + ((kj == ki) & lower).sum(-1)
        keep[r0:r0 + row_chunk] = (rank < n).reshape(-1, k)
    return keep


def sparsify(bits: np.ndarray, n: int, m: int):
    """S(X): kept values copied bit for bit, pruned values +0.0.  Returns (S bits, keep)."""
    keep = select_keep(bits, n, m)
    return np.where(keep, bits, np.uint16(0)).astype(np.uint16), keep


SCORE_ACT_WEIGHTED = 0   # score = |x_k| * c_k   (activation weighted by weight magnitude)
SCORE_WEIGHT = 1         # score = c_k           (weight magnitude alone)


def selection_scores(bits: np.ndarray, col_score: np.ndarray, mode: int) -> np.ndarray:
    """Per-element selection scores of the alternative strategies.  [FLEX] 2.A lists,
    besides ACT, a weight-magnitude score (WT) and Amber-Pruner, which weights the
    activation importance by the magnitude of the corresponding weights.

    col_score: fp32 [K], c_k >= 0 finite: a per-input-channel weight magnitude supplied by
    the caller (the pages do not fix the statistic or its outlier handling).
      mode SCORE_ACT_WEIGHTED: s = fp32(|x|) * c_k, one fp32 multiply (round to nearest
                               even, subnormals kept), as the GPU computes it;
      mode SCORE_WEIGHT:       s = c_k for every row.
    x must be finite.  Returns fp32 [R][K]."""
    bits = np.asarray(bits, dtype=np.uint16)
    c = np.asarray(col_score, dtype=np.float32)
    if c.shape != (bits.shape[1],):
        raise ValueError("col_score must have one entry per column")
    if mode == SCORE_WEIGHT:
        return np.broadcast_to(c, bits.shape).copy()
    if mode != SCORE_ACT_WEIGHTED:
        raise ValueError("unknown score mode")
    mag = ((bits & np.uint16(0x7FFF)).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return (mag * c[None, :]).astype(np.float32)


def select_keep_scored(bits: np.ndarray, col_score: np.ndarray, n: int, m: int, mode: int,
                       row_chunk: int = 256) -> np.ndarray:
    """Keep mask of the per-group top-n by selection score (selection_scores): the same
    rank rule as select_keep with the score in place of the magnitude,
        rank_i = #{j : s_j > s_i} + #{j < i : s_j == s_i},  keep iff rank_i < n."""
    if not (1 <= n <= m):
        raise ValueError("need 1 <= n <= m")
    score = selection_scores(bits, col_score, mode)
    r, k = score.shape
    if k % m:
        raise ValueError("K must be a multiple of m")
    keep = np.empty((r, k), dtype=bool)
    lower = np.tril(np.ones((m, m), dtype=bool), k=-1)
    for r0 in range(0, r, row_chunk):
        sc = score[r0:r0 + row_chunk].reshape(-1, k // m, m)
        si = sc[..., :, None]
        sj = sc[..., None, :]
        rank = (sj > si).sum(-1) + ((sj == si) & lower).sum(-1)
        keep[r0:r0 + row_chunk] = (rank < n).reshape(-1, k)
    return keep


def sparsify_scored(bits: np.ndarray, col_score: np.ndarray, n: int, m: int, mode: int):
    """S(X) under a scored selection: kept values bit for bit, pruned +0.0."""
    keep = select_keep_scored(bits, col_score, n, m, mode)
    return np.where(keep, np.asarray(bits, dtype=np.uint16), np.uint16(0)).astype(np.uint16), keep


def pack_mask(keep: np.ndarray) -> np.ndarray:
    """Bitmask words: word [r][k // 32], bit (k % 32) set iff position k is kept."""
    r, k = keep.shape
    words = (k + 31) // 32
    out = np.zeros((r, words), dtype=np.uint32)
    for kk in range(k):
        out[:, kk // 32] |= keep[:, kk].astype(np.uint32) << np.uint32(kk % 32)
    return out


def compress(bits: np.ndarray, n: int, m: int):
    """Compressed form: values [R][K*n/m] (kept values of each group in ascending
    position) and idx [R][K*n/m] uint8 (their in-group positions).  [FLEX] section 1
    (values plus index metadata)."""
    keep = select_keep(bits, n, m)
    r, k = bits.shape
    g = k // m
    pos = np.broadcast_to(np.arange(m), (r, g, m))
    kg = keep.reshape(r, g, m)
    # each group holds exactly n kept positions; boolean indexing keeps ascending order
    idx = pos[kg].reshape(r, g * n).astype(np.uint8)
    vals = bits.reshape(r, g, m)[kg].reshape(r, g * n).astype(np.uint16)
    return vals, idx


def pack_meta_2bit(idx: np.ndarray) -> np.ndarray:
    """2:4 metadata, two bits per kept value: slot j -> byte j // 4, bits 2*(j % 4)."""
    r, s = idx.shape
    out = np.zeros((r, (s + 3) // 4), dtype=np.uint8)
    for j in range(s):
        if np.any(idx[:, j] > 3):
            raise ValueError("2-bit metadata needs positions < 4")
        out[:, j // 4] |= (idx[:, j].astype(np.uint8) << np.uint8(2 * (j % 4)))
    return out


def unpack_meta_2bit(meta: np.ndarray, slots: int) -> np.ndarray:
    r = meta.shape[0]
    out = np.zeros((r, slots), dtype=np.uint8)
    for j in range(slots):
        out[:, j] = (meta[:, j // 4] >> np.uint8(2 * (j % 4))) & np.uint8(3)
    return out


def decompress(vals: np.ndarray, idx: np.ndarray, n: int, m: int, k: int) -> np.ndarray:
    """Inverse of compress: scatter value slot (g, i) to position g*m + idx, +0.0 elsewhere."""
    r = vals.shape[0]
    g = k // m
    out = np.zeros((r, k), dtype=np.uint16)
    v = vals.reshape(r, g, n)
    ix = idx.reshape(r, g, n).astype(np.int64)
    base = (np.arange(g) * m)[None, :, None]
    rows = np.arange(r)[:, None, None]
    out[np.broadcast_to(rows, ix.shape), base + ix] = v
    return out


# ---------------------------------------------------------------------- slide (6:8) ---

def lowered_k(k: int, ns: int) -> int:
    """K' = K * (2N-2)/N: each group of 2N positions becomes N-1 windows of 4.
    [SLIDE] 2.A (expansion factor gamma)."""
    if k % (2 * ns):
        raise ValueError("K must be a multiple of 2N")
    return (k // (2 * ns)) * 4 * (ns - 1)


def slide_windows(kept_positions, ns: int):
    """Assign the kept positions of one group of 2N to the N-1 windows
    (window w covers positions 2w .. 2w+3).  Returns a list of per-window position lists.
    [SLIDE] 2.A: visit kept positions in ascending order, each to the lowest covering
    window still holding fewer than two; overflow moves to the next window."""
    windows = [[] for _ in range(ns - 1)]
    for p in sorted(kept_positions):
        placed = False
        for w in range(ns - 1):
            if 2 * w <= p <= 2 * w + 3 and len(windows[w]) < 2:
                windows[w].append(p)
                placed = True
                break
        if not placed:
            raise ValueError(f"position {p} cannot be placed: not a (2N-2):2N group")
    return windows


def slide_lower(vals: np.ndarray, idx: np.ndarray, k: int, ns: int):
    """Offline packer: a (2N-2):2N matrix given as (values, u8 idx) -> the lowered 2:4
    matrix over K' (values [R][K'/2], idx [R][K'/2] with in-window slots 0..3).
    [SLIDE] 2.A, 2.C.  Window w of group g holds lowered positions g*4(N-1)+4w+s."""
    n = 2 * ns - 2
    m = 2 * ns
    r = vals.shape[0]
    g_count = k // m
    kp = lowered_k(k, ns)
    out_v = np.zeros((r, kp // 2), dtype=np.uint16)
    out_i = np.zeros((r, kp // 2), dtype=np.uint8)
    for row in range(r):
        for g in range(g_count):
            pos = [int(p) for p in idx[row, g * n:(g + 1) * n]]
            val = [vals[row, g * n + j] for j in range(n)]
            byp = dict(zip(pos, val))
            wins = slide_windows(pos, ns)
            for w, plist in enumerate(wins):
                if len(plist) != 2:
                    raise ValueError("window not filled with exactly two")
                for j, p in enumerate(plist):      # ascending in-window slot order
                    slot = (g * (ns - 1) + w) * 2 + j
                    out_v[row, slot] = byp[p]
                    out_i[row, slot] = p - 2 * w
    return out_v, out_i


def slide_scatter_back(vals_p: np.ndarray, idx_p: np.ndarray, k: int, ns: int) -> np.ndarray:
    """Sum the windows back onto the original 2N positions (dense bf16 bits [R][K]).
    Each original position receives at most one window entry."""
    r = vals_p.shape[0]
    out = np.zeros((r, k), dtype=np.uint16)
    filled = np.zeros((r, k), dtype=bool)
    wcount = (k // (2 * ns)) * (ns - 1)
    for row in range(r):
        for wi in range(wcount):
            g, w = divmod(wi, ns - 1)
            for j in range(2):
                slot = wi * 2 + j
                p = g * 2 * ns + 2 * w + int(idx_p[row, slot])
                if filled[row, p]:
                    raise ValueError("two windows claim one position")
                filled[row, p] = True
                out[row, p] = vals_p[row, slot]
    return out


def lift(x_bits: np.ndarray, ns: int) -> np.ndarray:
    """Activation lifting: X'[t][g*4(N-1) + 4w + s] = X[t][g*2N + 2w + s].  [SLIDE] 2.B."""
    t, k = x_bits.shape
    kp = lowered_k(k, ns)
    out = np.empty((t, kp), dtype=np.uint16)
    for kk in range(kp):
        g, rem = divmod(kk, 4 * (ns - 1))
        w, s = divmod(rem, 4)
        out[:, kk] = x_bits[:, g * 2 * ns + 2 * w + s]
    return out


# -------------------------------------------------------------------------- hybrid ---

def column_sq_norms(w_bits: np.ndarray) -> np.ndarray:
    """c_k = sum over o (ascending) of W[o][k]^2 in fp64 (squares of bf16 are exact)."""
    w = bf16_to_f64(w_bits)
    c = np.zeros(w.shape[1], dtype=np.float64)
    for o in range(w.shape[0]):
        c = c + w[o] * w[o]
    return c


def hybrid_columns(w_bits: np.ndarray, k_dense: int):
    """[SPENSE] 2.A/2.B: choose the dense columns (largest L2 norm, ties to the lower
    column) and order the sparse region first, dense region second, each ascending."""
    c = column_sq_norms(w_bits)
    k = c.shape[0]
    order = sorted(range(k), key=lambda j: (-c[j], j))
    dense = np.array(sorted(order[:k_dense]), dtype=np.int32)
    is_dense = np.zeros(k, dtype=bool)
    is_dense[dense] = True
    sparse = np.array([j for j in range(k) if not is_dense[j]], dtype=np.int32)
    return sparse, dense


def hybrid_pack(w_bits: np.ndarray, k_dense: int):
    """Offline hybrid packing: (sparse_cols, dense_cols, W_s values, W_s idx, W_d)."""
    sparse, dense = hybrid_columns(w_bits, k_dense)
    ws = np.ascontiguousarray(w_bits[:, sparse])
    wd = np.ascontiguousarray(w_bits[:, dense])
    if ws.shape[1]:
        v, i = compress(ws, 2, 4)
    else:
        v = np.zeros((w_bits.shape[0], 0), np.uint16)
        i = np.zeros((w_bits.shape[0], 0), np.uint8)
    return sparse, dense, v, i, wd


# -------------------------------------------------------------- Spense GLU (MLP) ---
# [SPENSE] 2.A: output-split for the gate and up projections (rows split between a 2:4
# GEMM and a dense GEMM), input-split for the down projection; 2.B: the intermediate
# indices of a GLU MLP can be permuted without changing its result, so the dense ones are
# chosen by a score and moved into one contiguous block.

def spense_glu_scores(w_gate, w_up, w_down, hs_in, hs_mid) -> np.ndarray:
    """Loss-aware importance of each intermediate index i ([SPENSE] 2.B, the "+" strategy):
    the Wanda-style score |W_ij| * sqrt(H_jj) summed over the three projections that touch
    index i.  Reading (the page gives the per-weight score and says it is aggregated over
    gate, up and down, nothing more):
        g_i = sum_j |W_gate[i][j]| * hs_in[j]     (j ascending)
        u_i = sum_j |W_up[i][j]|   * hs_in[j]     (j ascending)
        d_i = sum_o |W_down[o][i]|                (o ascending)
        S_i = (g_i + u_i) + hs_mid[i] * d_i
    in fp64, every product and sum rounded once in that order; hs_in / hs_mid are the
    square roots of the input Hessian diagonals (X^T X over calibration tokens), given by
    the caller.  w_*: bf16 bits, gate/up [I][H], down [H][I]."""
    g = np.abs(bf16_to_f64(w_gate)) * np.asarray(hs_in, np.float64)[None, :]
    u = np.abs(bf16_to_f64(w_up)) * np.asarray(hs_in, np.float64)[None, :]
    d = np.abs(bf16_to_f64(w_down))
    gs = np.cumsum(g, axis=1)[:, -1] if g.shape[1] else np.zeros(g.shape[0])   # left-to-right
    us = np.cumsum(u, axis=1)[:, -1] if u.shape[1] else np.zeros(u.shape[0])
    ds = np.cumsum(d, axis=0)[-1] if d.shape[0] else np.zeros(d.shape[1])
    return (gs + us) + np.asarray(hs_mid, np.float64) * ds


def spense_order(scores: np.ndarray, n_dense: int) -> np.ndarray:
    """Permutation of the intermediate indices: the n_dense largest scores (ties to the
    lower index) are dense; sparse indices first, then dense ones, each ascending."""
    i_n = len(scores)
    order = sorted(range(i_n), key=lambda j: (-scores[j], j))
    dense = sorted(order[:n_dense])
    is_dense = np.zeros(i_n, dtype=bool)
    is_dense[dense] = True
    return np.array([j for j in range(i_n) if not is_dense[j]] + dense, dtype=np.int32)


def spense_order_tail(i_n: int, n_dense: int) -> np.ndarray:
    """The simple strategy ([SPENSE] 2.B): the last n_dense indices stay dense (identity)."""
    return np.arange(i_n, dtype=np.int32)


def spense_pack(w_bits, perm, n_sparse: int, axis: int):
    """Split a weight along `axis` by the permutation: axis 0 (output-split) takes rows
    perm[:n_sparse] as the 2:4 region (pruned and compressed along K) and rows
    perm[n_sparse:] as the dense region; axis 1 (input-split) does the same with columns.
    Returns (W_s values, W_s idx, W_d)."""
    w = np.asarray(w_bits, dtype=np.uint16)
    perm = np.asarray(perm, dtype=np.int64)
    if axis == 0:
        ws, wd = w[perm[:n_sparse]], w[perm[n_sparse:]]
    else:
        ws, wd = w[:, perm[:n_sparse]], w[:, perm[n_sparse:]]
    ws, wd = np.ascontiguousarray(ws), np.ascontiguousarray(wd)
    if ws.size:
        v, i = compress(ws, 2, 4)
    else:
        v = np.zeros((ws.shape[0], ws.shape[1] // 2), np.uint16)
        i = np.zeros((ws.shape[0], ws.shape[1] // 2), np.uint8)
    return v, i, wd


def outsplit_gemm(x_bits, ws_vals, ws_idx, wd_bits, k: int) -> np.ndarray:
    """[SPENSE] 2.A output split: Y = [X . W_s^T, X . W_d^T] (W_s 2:4 compressed rows)."""
    parts = []
    if ws_vals.shape[0]:
        parts.append(gemm(x_bits, decompress(ws_vals, ws_idx, 2, 4, k)))
    if wd_bits.shape[0]:
        parts.append(gemm(x_bits, wd_bits))
    return np.concatenate(parts, axis=1)


# ---------------------------------------------------------------------------- GEMM ---

_HERE = os.path.dirname(os.path.abspath(__file__))
_C_SRC = os.path.join(_HERE, "gemm_f32.c")
_C_LIB = os.path.join(_HERE, "liboracle.so")
# plain C, no fused multiply-add contraction, no fast-math reassociation
_C_FLAGS = ["-O3", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off", "-fno-fast-math"]
_clib_handle = None


def build_c() -> str:
    """Compile the oracle's C part (gemm_f32.c) into oracle/liboracle.so with gcc."""
    tmp = _C_LIB + ".tmp"
    subprocess.run(["gcc", *_C_FLAGS, _C_SRC, "-o", tmp], check=True)
    os.replace(tmp, _C_LIB)
    return _C_LIB


def _clib():
    global _clib_handle
    if _clib_handle is None:
        if not os.path.exists(_C_LIB) or os.path.getmtime(_C_LIB) < os.path.getmtime(_C_SRC):
            build_c()
        lib = ctypes.CDLL(_C_LIB)
        lib.oracle_gemm_f32.restype = None
        lib.oracle_gemm_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]
        _clib_handle = lib
    return _clib_handle


def gemm_f32_values(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y[t][o] = fp32 sum over ascending k of a[t][k] * b[o][k], one accumulator per output
    starting at +0, every sum rounded to nearest even (gemm_f32.c).  a: fp32 [T][K],
    b: fp32 [O][K] holding values whose pairwise products are exact in fp32 (bf16, e4m3).
    Returns fp32 [T][O]."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    t, k = a.shape
    o = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("operands disagree on K")
    bk = np.ascontiguousarray(b.T)            # K-major: one k's weights contiguous
    y = np.empty((t, o), dtype=np.float32)
    if t and o:
        _clib().oracle_gemm_f32(a.ctypes.data, t, k, bk.ctypes.data, o, y.ctypes.data)
    return y


def gemm(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Y[t][o] = sum over ascending k of a[t][k] * b[o][k], accumulated in fp32 (the
    layer's "fp32 accumulate"; gemm_f32_values).  bf16 operands; returns the fp32 results
    as fp64 values."""
    return gemm_f32_values(f32_from_bf16(a_bits), f32_from_bf16(b_bits)).astype(np.float64)


def gemm_f64(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """The same product in fp64 (library matrix product): error bounds and projection
    checks only."""
    return bf16_to_f64(a_bits) @ bf16_to_f64(b_bits).T


def spmm_act(x_bits: np.ndarray, w_bits: np.ndarray, n: int, m: int) -> np.ndarray:
    """Activation-sparse layer Y = S(X) . W^T.  [FLEX] 2.A, 2.C."""
    s, _ = sparsify(x_bits, n, m)
    return gemm(s, w_bits)


def spmm_slide(x_bits: np.ndarray, vals_p: np.ndarray, idx_p: np.ndarray, ns: int) -> np.ndarray:
    """Lowered weight-sparse layer Y = lift(X) . W'^T.  [SLIDE] 2.A-2.C."""
    k = x_bits.shape[1]
    kp = lowered_k(k, ns)
    wp = decompress(vals_p, idx_p, 2, 4, kp)
    return gemm(lift(x_bits, ns), wp)


def hybrid_gemm(x_bits, sparse_cols, dense_cols, ws_vals, ws_idx, wd_bits) -> np.ndarray:
    """[SPENSE] 2.A input split: Y = X_s . W_s^T + X_d . W_d^T, where X_s / X_d are the
    columns of X in the sparse / dense region order and W_s is 2:4 compressed.  One fp32
    accumulator per output runs over the sparse region, then the dense region."""
    ks = len(sparse_cols)
    o = wd_bits.shape[0] if wd_bits.size else ws_vals.shape[0]
    a_parts = [np.asarray(x_bits)[:, np.asarray(sparse_cols, np.int64)],
               np.asarray(x_bits)[:, np.asarray(dense_cols, np.int64)]]
    b_parts = [decompress(ws_vals, ws_idx, 2, 4, ks) if ks else np.zeros((o, 0), np.uint16),
               np.asarray(wd_bits, np.uint16).reshape(o, len(dense_cols))]
    # one accumulator per output: the sparse region's products first, then the dense region's
    return gemm(np.concatenate(a_parts, axis=1), np.concatenate(b_parts, axis=1))


# ----------------------------------------------------------------------------- fp8 ---

def fp8_e4m3_to_f64(q: np.ndarray) -> np.ndarray:
    """OCP E4M3FN decode: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity."""
    q = np.asarray(q, dtype=np.uint8).astype(np.int64)
    s = np.where(q >> 7, -1.0, 1.0)
    e = (q >> 3) & 15
    mant = q & 7
    normal = s * np.ldexp(1.0 + mant / 8.0, e - 7)
    sub = s * mant * 2.0 ** -9
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (mant == 7), np.nan, out)


E4M3_MAX = 448.0


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Values with |v| <= 448 -> OCP E4M3FN codes, round to nearest, ties to even.
    Normal range (|v| >= 2^-6): v = 2^e (1 + f), f rounded to 3 bits (a carry moves to the
    next exponent); below it the subnormal step 2^-9 (q = round(|v| / 2^-9), and q = 8 is the
    smallest normal, code 0x08).  Zero encodes as 0x00 (+0) or 0x80 (-0)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode needs finite |v| <= 448")
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    mant, ex = np.frexp(a)                      # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                  # a = (2 mant) * 2^e, 2 mant in [1, 2)
    f8 = np.rint((2.0 * mant - 1.0) * 8.0)      # 3 fraction bits, ties to even (exact in fp64)
    carry = f8 == 8.0
    e = np.where(carry, e + 1, e)
    f8 = np.where(carry, 0.0, f8)
    normal = ((e + 7) << 3).astype(np.int64) + f8.astype(np.int64)
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)   # 0..8; 8 is code 0x08, the smallest normal
    code = np.where(a >= 2.0 ** -6, normal, sub)
    return (code | sign).astype(np.uint8)


def quantize_tokens(x_bits: np.ndarray):
    """Per-token fp8 quantization of bf16 activations (the online step of the SlideSparse
    page, technical summary 2.B, which fuses it with the lift; the page gives no scheme).
    Reading: symmetric absmax scaling to the e4m3 range, per row t:
        amax_t = max_k |x_tk|;  r_t = fp32(448 / amax_t);  s_t = fp32(amax_t / 448)
        q_tk  = e4m3_encode(clamp(fp32(x_tk * r_t), -448, 448))
    with r_t = s_t = 1 for an all-zero row; every fp32 operation rounds to nearest even.
    Parity unpinned in the multiply-by-r reading (x / s is as plain; see the header).
    Returns (codes uint8 [T][K], scales fp32 [T]); x ~= dec(q) * s."""
    x = f32_from_bf16(x_bits)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    r = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    s = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    v = (x * r[:, None]).astype(np.float32)
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(v), s


def f32_from_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def spmm_w8a8_slide(x_bits, w8_vals, w_idx, w_scale, k: int, ns: int) -> np.ndarray:
    """fp8 weights and fp8 activations (the SlideSparse page's serving precision, technical
    summary 2.B-2.C): X quantized per token, lifted ((2N-2):2N weights lowered to 2:4 over
    K' = K (2N-2)/N; ns = 2 means plain 2:4, no lift), multiplied against the 2:4 weight
    codes W' (values [O][K'/2] + in-window positions), then both scales applied:
        Y[t][o] = fp32(fp32(s_t * sum_k' dec(lift(q)[t][k']) * dec(W'[o][k'])) * s_o)
    with the sum accumulated in fp32 in ascending k'."""
    q, s_t = quantize_tokens(x_bits)
    qx = lift(q, ns) if ns > 2 else q
    kp = qx.shape[1]
    wd = decompress(np.asarray(w8_vals, np.uint8).astype(np.uint16), w_idx, 2, 4, kp)
    # e4m3 x e4m3 products are exact in fp32; fp32 accumulation, then the two scales
    acc = gemm_f32_values(fp8_e4m3_to_f64(qx).astype(np.float32),
                          fp8_e4m3_to_f64(wd.astype(np.uint8)).astype(np.float32))
    y = (acc * s_t.astype(np.float32)[:, None]).astype(np.float32)
    return (y * np.asarray(w_scale, np.float32)[None, :]).astype(np.float32).astype(np.float64)


def spmm_act_fp8(x_bits: np.ndarray, w8: np.ndarray, scale: np.ndarray, n: int, m: int) -> np.ndarray:
    """Y[t][o] = fp32(scale[o] * sum_k S(X)[t][k] * dec(W8[o][k])): the sum accumulated in
    fp32 in ascending k, the scale applied once after it."""
    s, _ = sparsify(x_bits, n, m)
    # bf16 x e4m3 products are exact in fp32; fp32 accumulation, then one scale multiply
    acc = gemm_f32_values(f32_from_bf16(s), fp8_e4m3_to_f64(w8).astype(np.float32))
    return (acc * np.asarray(scale, dtype=np.float32)[None, :]).astype(np.float32).astype(np.float64)


# ---------------------------------------------------- error mitigation (PTS, VAR) ---
# [FLEX] technical summary 2.B lists light-weight corrections of the pruning error that need
# little or no calibration: a per-token shift that centres the activations around zero
# before pruning, dynamic (D-PTS: computed from each token) or static (S-PTS: fixed in
# advance), and VAR, a per-token correction of the variance after pruning; 4.C ranks them
# among the most effective.  The page gives no formulas.  Readings (the plainest ones):
#   D-PTS  mu_t = mean_k x_tk (reproducible, see pts_row_mean); prune x - mu_t; the shift is
#          undone after the product by the rank-one term mu_t * (W . 1)_o
#   S-PTS  a caller-given static shift c_k per input channel (a scalar shift is c_k = s);
#          prune x - c; undone by the constant term (W . c)_o
#   VAR    alpha_t = sqrt(Var(x~_t) / Var(S(x~_t))), Var = mean of squared deviations over
#          the row's K entries (pruned entries count as zeros); the pruned row is scaled
#          by alpha_t, so its variance equals the unpruned (shifted) row's
# With x~ = the shifted row, Y[t][o] = alpha_t * sum_k S(x~)[t][k] W[o][k] + beta_t v_o,
# beta_t = mu_t (D-PTS) or 1 (S-PTS), v = W . 1 or W . c; without a shift the last term is 0.

PTS_DYNAMIC = 1   # per-token shift by the row mean
PTS_STATIC = 2    # per-channel shift given by the caller
PTS_VAR = 4       # variance correction after pruning


def bf16_from_f32_rne(v: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even (finite and infinite
    inputs; a value rounding past the largest bf16 becomes infinity)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def pts_row_mean(x_bits: np.ndarray) -> np.ndarray:
    """D-PTS shift: the mean of each row, computed so that its bits do not depend on the
    order of summation (the selection that follows compares bits, so every implementation
    must reach the same mu).  Per row of finite bf16 values:
        E   = exponent field of M = max_k |x_k| (1 if M is subnormal);  M < 2^(E-126)
        q   = 2^(E - 162)                  every |x_k| / q < 2^36
        n_k = round-half-even(x_k / q)     an integer; exact for every x_k >= 2^(E-159)
        S   = sum_k n_k                    exact (|S| < 2^52 for K <= 2^16)
        mu  = fp32( fp64(S * q) / K )      one fp64 division, one rounding to fp32
    i.e. the exact mean of the row after rounding each value to a multiple of q (at most
    2^-37 M from the exact mean), rounded once.  mu = +0 for an all-zero row.  Returns fp32 [R]."""
    bits = np.asarray(x_bits, dtype=np.uint16)
    r, k = bits.shape
    if k > 65536:
        raise ValueError("rows longer than 65536")
    key = (bits & np.uint16(0x7FFF)).astype(np.int64)
    if np.any(key >= 0x7F80):
        raise ValueError("the shift needs finite activations")
    out = np.zeros(r, dtype=np.float32)
    vals = bf16_to_f64(bits)
    for row in range(r):
        m = int(key[row].max()) if k else 0
        if m == 0:
            continue
        e = max(m >> 7, 1)
        n = np.rint(np.ldexp(vals[row], 162 - e)).astype(np.int64)   # x / q, exact; then RNE
        total = 0
        for v in n.tolist():            # plain integer sum, ascending k (any order is exact)
            total += v
        mean = np.ldexp(float(total), e - 162) / float(k)
        out[row] = np.float32(mean)
    return out


def pts_shift(x_bits: np.ndarray, shift_rows=None, shift_cols=None) -> np.ndarray:
    """x~ = bf16( fp32(x - shift) ), both roundings to nearest even: shift_rows fp32 [R]
    (D-PTS, one value per token) or shift_cols fp32 [K] (S-PTS, one per channel)."""
    x = f32_from_bf16(x_bits)
    if shift_rows is not None:
        d = (x - np.asarray(shift_rows, np.float32)[:, None]).astype(np.float32)
    elif shift_cols is not None:
        d = (x - np.asarray(shift_cols, np.float32)[None, :]).astype(np.float32)
    else:
        return np.asarray(x_bits, dtype=np.uint16).copy()
    return bf16_from_f32_rne(d)


def var_scale(xs_bits: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """VAR: alpha_t = sqrt(Var(x~_t) / Var(S(x~_t))) over the K entries of each row (mean of
    squared deviations from the row mean, fp64, two passes), alpha = 1 when the pruned row
    has no variance.  Returns fp32 [R]."""
    a = bf16_to_f64(xs_bits)
    b = bf16_to_f64(s_bits)
    va = ((a - a.mean(axis=1, keepdims=True)) ** 2).mean(axis=1) if a.shape[1] else np.zeros(a.shape[0])
    vb = ((b - b.mean(axis=1, keepdims=True)) ** 2).mean(axis=1) if b.shape[1] else np.zeros(b.shape[0])
    alpha = np.ones(a.shape[0])
    ok = vb > 0
    alpha[ok] = np.sqrt(va[ok] / vb[ok])
    return alpha.astype(np.float32)


def sparsify_pts(x_bits: np.ndarray, n: int, m: int, mode: int, static_shift=None):
    """Shift (D-PTS or S-PTS, or none), select (the ACT rule on the shifted bf16 values) and
    optionally the VAR scale.  Returns (S(x~) bits, keep, mu fp32 [R] or None, alpha fp32 [R]
    or None).  mode: PTS_DYNAMIC or PTS_STATIC (not both), optionally | PTS_VAR."""
    if (mode & PTS_DYNAMIC) and (mode & PTS_STATIC):
        raise ValueError("one shift at a time")
    mu = None
    if mode & PTS_DYNAMIC:
        mu = pts_row_mean(x_bits)
        xs = pts_shift(x_bits, shift_rows=mu)
    elif mode & PTS_STATIC:
        xs = pts_shift(x_bits, shift_cols=np.asarray(static_shift, np.float32))
    else:
        xs = np.asarray(x_bits, dtype=np.uint16)
    s, keep = sparsify(xs, n, m)
    alpha = var_scale(xs, s) if mode & PTS_VAR else None
    return s, keep, mu, alpha


def weight_sums(w_vals: np.ndarray, shift=None) -> np.ndarray:
    """The term that undoes a shift after the product: v_o = sum_k W[o][k] * c_k (c = 1 for
    D-PTS, the static shift for S-PTS), summed in fp64 over ascending k and rounded once to
    fp32.  w_vals: fp64 weight values [O][K] (bf16, or fp8 codes times their row scale)."""
    w = np.asarray(w_vals, dtype=np.float64)
    c = np.ones(w.shape[1]) if shift is None else np.asarray(shift, np.float32).astype(np.float64)
    out = np.zeros(w.shape[0])
    for kk in range(w.shape[1]):
        out = out + w[:, kk] * c[kk]
    return out.astype(np.float32)


def spmm_pts(x_bits, w_bits, n: int, m: int, mode: int, static_shift=None, col_shift=None):
    """The mitigated layer: Y = alpha_t * (S(x~) . W^T) + beta_t * v_o with the product
    accumulated in fp32 (gemm) and the two terms added in fp64.  col_shift: v (fp32 [O]) as
    the caller supplies it (weight_sums of W, with the static shift for S-PTS).
    Returns (Y fp64, S(x~) bits, keep, mu, alpha)."""
    s, keep, mu, alpha = sparsify_pts(x_bits, n, m, mode, static_shift)
    y = gemm(s, w_bits)
    if alpha is not None:
        y = y * alpha.astype(np.float64)[:, None]
    if mode & (PTS_DYNAMIC | PTS_STATIC):
        v = np.asarray(col_shift, np.float32).astype(np.float64)[None, :]
        beta = mu.astype(np.float64)[:, None] if mode & PTS_DYNAMIC else 1.0
        y = y + beta * v
    return y, s, keep, mu, alpha
