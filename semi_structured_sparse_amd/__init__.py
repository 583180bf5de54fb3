"""Python binding of libnmsparse (N:M structured-sparse linear layers on MI355X / gfx950).

Thin ctypes layer: every function has the name of the C entry point it calls and only
marshals arguments (device pointers, sizes, leading dimensions, the current HIP stream).
All arithmetic runs in the library's HIP kernels.  torch tensors serve as device memory:
bf16 data may be any 2-byte dtype (torch.bfloat16, int16, uint16 holding bf16 bits).

The library must have been built (``semi_structured_sparse_amd.build.build()``); there is
no fallback: importing the binding without the shared library raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "NMError", "lib", "NM_OK", "NM_EINVAL", "NM_ESHAPE", "NM_EALIGN", "NM_EUNSUPPORTED", "NM_EHIP",
    "NM_META_U8", "NM_META_2BIT", "NM_W_BF16", "NM_W_FP8E4M3", "NM_ACT_DYNAMIC", "NM_ACT_COMPRESSED",
    "NM_W_COMPRESSED", "NM_W_SLIDE", "NM_ACT_MASKED", "nm_spmm_args", "nm_status_str", "nm_version", "nm_sparsify",
    "nm_sparsify_scored", "NM_SCORE_ACT_WEIGHTED", "NM_SCORE_WEIGHT", "route_taken", "ROUTE", "TAKEN",
    "route_bits", "taken_names", "make_spmm_args",
    "nm_compress", "nm_decompress", "nm_lower_slide", "nm_slide_lift", "nm_spmm",
    "nm_spmm_workspace_size", "nm_hybrid_pack", "nm_hybrid_pack_workspace_size", "nm_hybrid_gemm",
    "nm_hybrid_gemm_workspace_size", "lowered_k", "NM_SPENSE_LOSS", "NM_SPENSE_TAIL", "nm_spense_glu_order",
    "nm_spense_glu_order_workspace_size", "nm_spense_pack", "nm_spense_pack_workspace_size",
    "nm_spense_outsplit_gemm", "nm_spense_outsplit_workspace_size", "nm_quant_lift", "NM_PTS_DYNAMIC",
    "NM_PTS_STATIC", "NM_PTS_VAR", "nm_sparsify_pts", "nm_weight_sums", "NM_ESCRATCH", "nm_spmm_noalloc",
    "NM_NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnmsparse.so")

NM_OK, NM_EINVAL, NM_ESHAPE, NM_EALIGN, NM_EUNSUPPORTED, NM_EHIP, NM_ESCRATCH = range(7)
NM_NOALLOC_SCRATCH_BYTES = 64 << 20
NM_META_U8, NM_META_2BIT = 0, 1
NM_W_BF16, NM_W_FP8E4M3 = 0, 1
NM_SCORE_ACT_WEIGHTED, NM_SCORE_WEIGHT = 0, 1
NM_SPENSE_LOSS, NM_SPENSE_TAIL = 0, 1
NM_ACT_DYNAMIC, NM_ACT_COMPRESSED, NM_W_COMPRESSED, NM_W_SLIDE, NM_ACT_MASKED = range(5)
NM_PTS_DYNAMIC, NM_PTS_STATIC, NM_PTS_VAR = 1, 2, 4

# route hints (NM_ROUTE_*) and the report of what ran (NM_TAKEN_*), by lower-case name
ROUTE = {name: 1 << i for i, name in enumerate(
    ["act_fused", "act_mask", "act_sx", "no_few", "few_stream", "few_tile", "no_meta_block", "fp8_widen",
     "no_xlds", "no_few_select", "tile_lds", "tile_regs", "lift_copy", "act_sparse_x", "row_sx"])}
TAKEN = {name: 1 << i for i, name in enumerate(
    ["select", "few_stream", "few_xlds", "few_select", "tile_split", "reduce", "tile_lds", "tile_regs",
     "fused_select", "mask", "gather1", "lift", "meta_block", "permute", "quant", "widen", "decompress",
     "sparse_mma"])}


def route_bits(*names) -> int:
    """OR of the NM_ROUTE_* bits named (e.g. route_bits("few_stream", "no_xlds"))."""
    bits = 0
    for nm in names:
        bits |= ROUTE[nm]
    return bits


def taken_names(bits: int) -> set:
    """The NM_TAKEN_* names set in a route report."""
    return {nm for nm, b in TAKEN.items() if bits & b}


_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p


class nm_spmm_args(ctypes.Structure):
    _fields_ = [
        ("mode", _int), ("n", _int), ("m", _int), ("ns", _int),
        ("t", _i64), ("o", _i64), ("k", _i64),
        ("x", _vp), ("ldx", _i64), ("x_meta", _vp), ("x_meta_fmt", _int),
        ("w", _vp), ("ldw", _i64), ("w_dtype", _int), ("w_meta", _vp), ("w_meta_fmt", _int),
        ("w_scale", _vp), ("w_kmajor", _vp),
        ("y", _vp), ("ldy", _i64), ("accumulate", _int),
        ("x_mask_out", _vp), ("workspace", _vp), ("workspace_bytes", _i64),
        ("route", ctypes.c_uint32), ("few_wpb", ctypes.c_int32), ("few_splits", ctypes.c_int32),
        ("tile_wg", ctypes.c_int32), ("route_taken", _vp),
        ("pts", _int), ("pts_shift", _vp), ("col_shift", _vp), ("row_scale", _vp), ("row_shift", _vp),
    ]


class NMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {nm_status_str(status)}")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libnmsparse.so once; raise ImportError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with semi_structured_sparse_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.nm_status_str.restype = ctypes.c_char_p
    L.nm_status_str.argtypes = [_int]
    L.nm_version.restype = _int
    L.nm_version.argtypes = []
    L.nm_sparsify.restype = _int
    L.nm_sparsify.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _vp, _i64, _vp, _vp]
    L.nm_sparsify_scored.restype = _int
    L.nm_sparsify_scored.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _vp, _int, _vp, _i64, _vp, _vp]
    L.nm_sparsify_pts.restype = _int
    L.nm_sparsify_pts.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _i64, _vp, _vp, _vp, _vp]
    L.nm_weight_sums.restype = _int
    L.nm_weight_sums.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]
    L.nm_compress.restype = _int
    L.nm_compress.argtypes = [_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _int, _vp, _vp]
    L.nm_decompress.restype = _int
    L.nm_decompress.argtypes = [_vp, _vp, _int, _i64, _i64, _int, _int, _vp, _i64, _vp]
    L.nm_lower_slide.restype = _int
    L.nm_lower_slide.argtypes = [_vp, _vp, _i64, _i64, _int, _vp, _vp, _int, _vp]
    L.nm_slide_lift.restype = _int
    L.nm_slide_lift.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _i64, _vp]
    L.nm_spmm.restype = _int
    L.nm_spmm.argtypes = [ctypes.POINTER(nm_spmm_args), _vp]
    L.nm_spmm_noalloc.restype = _int
    L.nm_spmm_noalloc.argtypes = [ctypes.POINTER(nm_spmm_args), _vp]
    L.nm_spmm_workspace_size.restype = _i64
    L.nm_spmm_workspace_size.argtypes = [ctypes.POINTER(nm_spmm_args)]
    L.nm_hybrid_pack.restype = _int
    L.nm_hybrid_pack.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _int, _vp, _i64, _vp, _i64, _vp]
    L.nm_hybrid_pack_workspace_size.restype = _i64
    L.nm_hybrid_pack_workspace_size.argtypes = [_i64]
    L.nm_hybrid_gemm.restype = _int
    L.nm_hybrid_gemm.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _int, _vp, _i64, _i64, _vp,
                                 _i64, _int, _vp, _i64, ctypes.c_uint32, _vp, _vp]
    L.nm_hybrid_gemm_workspace_size.restype = _i64
    L.nm_hybrid_gemm_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _int, ctypes.c_uint32]
    L.nm_quant_lift.restype = _int
    L.nm_quant_lift.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp]
    L.nm_spense_glu_order.restype = _int
    L.nm_spense_glu_order.argtypes = [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _int, _vp, _vp, _vp,
                                      _i64, _vp]
    L.nm_spense_glu_order_workspace_size.restype = _i64
    L.nm_spense_glu_order_workspace_size.argtypes = [_i64]
    L.nm_spense_pack.restype = _int
    L.nm_spense_pack.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp, _int, _vp, _i64, _vp, _i64, _vp]
    L.nm_spense_pack_workspace_size.restype = _i64
    L.nm_spense_pack_workspace_size.argtypes = [_i64, _i64, _int, _i64]
    L.nm_spense_outsplit_gemm.restype = _int
    L.nm_spense_outsplit_gemm.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _int,
                                          _vp, _i64, _vp]
    L.nm_spense_outsplit_workspace_size.restype = _i64
    L.nm_spense_outsplit_workspace_size.argtypes = [_i64, _i64, _i64, _i64]
    _LIB = L
    return L


# ------------------------------------------------------------------- marshalling ---

def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Integers pass through as raw pointers."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ld(t, default=0):
    if t is None:
        return default
    if t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("innermost dimension must be contiguous")
        return t.stride(0)
    return default


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != NM_OK:
        raise NMError(status, where)


def nm_status_str(status: int) -> str:
    return lib().nm_status_str(int(status)).decode()


def nm_version() -> int:
    return int(lib().nm_version())


def lowered_k(k: int, ns: int) -> int:
    """Reduction length after (2N-2):2N -> 2:4 lowering: k * (2N-2) / N."""
    return (k // (2 * ns)) * 4 * (ns - 1)


# ------------------------------------------------------------------- entry points ---

def nm_sparsify(x, n, m, y=None, mask=None, stream=None, *, rows=None, k=None, ldx=None, ldy=None, check=True):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    st = lib().nm_sparsify(_ptr(x), rows, k, _ld(x) if ldx is None else ldx, n, m, _ptr(y),
                           _ld(y) if ldy is None else ldy, _ptr(mask), _stream(stream))
    if check:
        _check(st, "nm_sparsify")
    return st


def nm_sparsify_scored(x, n, m, col_score, mode=NM_SCORE_ACT_WEIGHTED, y=None, mask=None, stream=None, *,
                       rows=None, k=None, ldx=None, ldy=None, check=True):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    st = lib().nm_sparsify_scored(_ptr(x), rows, k, _ld(x) if ldx is None else ldx, n, m, _ptr(col_score), mode,
                                  _ptr(y), _ld(y) if ldy is None else ldy, _ptr(mask), _stream(stream))
    if check:
        _check(st, "nm_sparsify_scored")
    return st


def nm_sparsify_pts(x, n, m, pts, y, mask=None, shift=None, row_shift=None, row_scale=None, stream=None, *,
                    rows=None, k=None, ldx=None, ldy=None, check=True):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    st = lib().nm_sparsify_pts(_ptr(x), rows, k, _ld(x) if ldx is None else ldx, n, m, pts, _ptr(shift), _ptr(y),
                               _ld(y) if ldy is None else ldy, _ptr(mask), _ptr(row_shift), _ptr(row_scale),
                               _stream(stream))
    if check:
        _check(st, "nm_sparsify_pts")
    return st


def nm_weight_sums(w, out, w_dtype=NM_W_BF16, w_scale=None, shift=None, stream=None, *, o=None, k=None, ldw=None,
                   check=True):
    o = w.shape[0] if o is None else o
    k = w.shape[1] if k is None else k
    st = lib().nm_weight_sums(_ptr(w), o, k, _ld(w) if ldw is None else ldw, w_dtype, _ptr(w_scale), _ptr(shift),
                              _ptr(out), _stream(stream))
    if check:
        _check(st, "nm_weight_sums")
    return st


def nm_compress(x, n, m, values, meta, fmt=NM_META_U8, mask=None, stream=None, *, rows=None, k=None, ldx=None,
                check=True):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    st = lib().nm_compress(_ptr(x), rows, k, _ld(x) if ldx is None else ldx, n, m, _ptr(values), _ptr(meta), fmt,
                           _ptr(mask), _stream(stream))
    if check:
        _check(st, "nm_compress")
    return st


def nm_decompress(values, meta, fmt, rows, k, n, m, y, stream=None, *, ldy=None, check=True):
    st = lib().nm_decompress(_ptr(values), _ptr(meta), fmt, rows, k, n, m, _ptr(y), _ld(y) if ldy is None else ldy,
                             _stream(stream))
    if check:
        _check(st, "nm_decompress")
    return st


def nm_lower_slide(values, idx, rows, k, ns, values_out, meta_out, fmt=NM_META_2BIT, stream=None, *, check=True):
    st = lib().nm_lower_slide(_ptr(values), _ptr(idx), rows, k, ns, _ptr(values_out), _ptr(meta_out), fmt,
                              _stream(stream))
    if check:
        _check(st, "nm_lower_slide")
    return st


def nm_slide_lift(x, ns, x_out, stream=None, *, t=None, k=None, ldx=None, ldo=None, check=True):
    t = x.shape[0] if t is None else t
    k = x.shape[1] if k is None else k
    st = lib().nm_slide_lift(_ptr(x), t, k, _ld(x) if ldx is None else ldx, ns, _ptr(x_out),
                             _ld(x_out) if ldo is None else ldo, _stream(stream))
    if check:
        _check(st, "nm_slide_lift")
    return st


def nm_spmm(args: nm_spmm_args, stream=None, *, check=True):
    st = lib().nm_spmm(ctypes.byref(args), _stream(stream))
    if check:
        _check(st, "nm_spmm")
    return st


def nm_spmm_noalloc(args: nm_spmm_args, stream=None, *, check=True):
    """nm_spmm with the library's own scratch (args.workspace must be NULL, bytes 0)."""
    st = lib().nm_spmm_noalloc(ctypes.byref(args), _stream(stream))
    if check:
        _check(st, "nm_spmm_noalloc")
    return st


def nm_spmm_workspace_size(args: nm_spmm_args) -> int:
    return int(lib().nm_spmm_workspace_size(ctypes.byref(args)))


def make_spmm_args(mode, t, o, k, x, w, y, *, n=2, m=4, ns=2, ldx=None, x_meta=None, x_meta_fmt=NM_META_U8,
                   ldw=None, w_dtype=NM_W_BF16, w_meta=None, w_meta_fmt=NM_META_2BIT, w_scale=None,
                   w_kmajor=None, ldy=None, accumulate=0, x_mask_out=None, workspace=None, workspace_bytes=0,
                   route=0, few_wpb=0, few_splits=0, tile_wg=0, pts=0, pts_shift=None, col_shift=None,
                   row_scale=None, row_shift=None):
    """Fill an nm_spmm_args from tensors (pointers and leading dimensions only).  The
    returned struct keeps references to the tensors so that their memory stays allocated
    while the struct is alive (it holds raw device pointers), and carries a report cell
    that route_taken(args) reads after a call."""
    a = nm_spmm_args()
    a._taken = ctypes.c_uint32(0)
    a.route, a.few_wpb, a.few_splits, a.tile_wg = route, few_wpb, few_splits, tile_wg
    a.route_taken = ctypes.addressof(a._taken)
    a._tensors = [v for v in (x, w, y, x_meta, w_meta, w_scale, w_kmajor, x_mask_out, workspace, pts_shift,
                              col_shift, row_scale, row_shift)
                  if v is not None and not isinstance(v, int)]
    a.pts, a.pts_shift, a.col_shift = pts, _ptr(pts_shift), _ptr(col_shift)
    a.row_scale, a.row_shift = _ptr(row_scale), _ptr(row_shift)
    a.mode, a.n, a.m, a.ns = mode, n, m, ns
    a.t, a.o, a.k = t, o, k
    a.x, a.ldx = _ptr(x), (_ld(x) if ldx is None else ldx)
    a.x_meta, a.x_meta_fmt = _ptr(x_meta), x_meta_fmt
    a.w, a.ldw, a.w_dtype = _ptr(w), (_ld(w) if ldw is None else ldw), w_dtype
    a.w_meta, a.w_meta_fmt = _ptr(w_meta), w_meta_fmt
    a.w_scale, a.w_kmajor = _ptr(w_scale), _ptr(w_kmajor)
    a.y, a.ldy, a.accumulate = _ptr(y), (_ld(y) if ldy is None else ldy), accumulate
    a.x_mask_out = _ptr(x_mask_out)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace_bytes
    return a


def nm_hybrid_pack(w, k_dense, sparse_cols, dense_cols, ws_values, ws_meta, fmt, wd, workspace, stream=None, *,
                   o=None, k=None, ldw=None, ldwd=None, workspace_bytes=None, check=True):
    o = w.shape[0] if o is None else o
    k = w.shape[1] if k is None else k
    wsb = (workspace.numel() * workspace.element_size()) if workspace_bytes is None else workspace_bytes
    st = lib().nm_hybrid_pack(_ptr(w), o, k, _ld(w) if ldw is None else ldw, k_dense, _ptr(sparse_cols),
                              _ptr(dense_cols), _ptr(ws_values), _ptr(ws_meta), fmt, _ptr(wd),
                              _ld(wd) if ldwd is None else ldwd, _ptr(workspace), wsb, _stream(stream))
    if check:
        _check(st, "nm_hybrid_pack")
    return st


def nm_hybrid_pack_workspace_size(k: int) -> int:
    return int(lib().nm_hybrid_pack_workspace_size(k))


def route_taken(args: nm_spmm_args) -> int:
    """NM_TAKEN_* bits reported by the calls made with args (made by make_spmm_args)."""
    return int(args._taken.value)


def nm_hybrid_gemm_workspace_size(t: int, k_s: int, k_d: int, o: int, gathered: bool, route: int = 0) -> int:
    return int(lib().nm_hybrid_gemm_workspace_size(t, k_s, k_d, o, 1 if gathered else 0, route))


def nm_quant_lift(x, ns, xq, xs, stream=None, *, t=None, k=None, ldx=None, ldq=None, check=True):
    t = x.shape[0] if t is None else t
    k = x.shape[1] if k is None else k
    st = lib().nm_quant_lift(_ptr(x), t, k, _ld(x) if ldx is None else ldx, ns, _ptr(xq),
                             _ld(xq) if ldq is None else ldq, _ptr(xs), _stream(stream))
    if check:
        _check(st, "nm_quant_lift")
    return st


def nm_spense_glu_order(w_gate, w_up, w_down, hs_in, hs_mid, n_dense, strategy, perm, workspace, scores=None,
                        stream=None, *, hidden=None, inter=None, ld_gu=None, ld_d=None, workspace_bytes=None,
                        check=True):
    inter = (w_gate.shape[0] if w_gate is not None else perm.shape[0]) if inter is None else inter
    hidden = (w_gate.shape[1] if w_gate is not None else 0) if hidden is None else hidden
    wsb = (workspace.numel() * workspace.element_size()) if workspace_bytes is None else workspace_bytes
    st = lib().nm_spense_glu_order(_ptr(w_gate), _ptr(w_up), (_ld(w_gate) if w_gate is not None else 0)
                                   if ld_gu is None else ld_gu, _ptr(w_down),
                                   (_ld(w_down) if w_down is not None else 0) if ld_d is None else ld_d, hidden,
                                   inter, _ptr(hs_in), _ptr(hs_mid), n_dense, strategy, _ptr(perm), _ptr(scores),
                                   _ptr(workspace), wsb, _stream(stream))
    if check:
        _check(st, "nm_spense_glu_order")
    return st


def nm_spense_glu_order_workspace_size(inter: int) -> int:
    return int(lib().nm_spense_glu_order_workspace_size(inter))


def nm_spense_pack(w, axis, perm, n_sparse, ws_values, ws_meta, fmt, wd, workspace=None, stream=None, *, o=None,
                   k=None, ldw=None, ldwd=None, workspace_bytes=None, check=True):
    o = w.shape[0] if o is None else o
    k = w.shape[1] if k is None else k
    wsb = (workspace.numel() * workspace.element_size() if workspace is not None else 0) \
        if workspace_bytes is None else workspace_bytes
    st = lib().nm_spense_pack(_ptr(w), o, k, _ld(w) if ldw is None else ldw, axis, _ptr(perm), n_sparse,
                              _ptr(ws_values), _ptr(ws_meta), fmt, _ptr(wd),
                              (_ld(wd) if wd is not None else 0) if ldwd is None else ldwd, _ptr(workspace), wsb,
                              _stream(stream))
    if check:
        _check(st, "nm_spense_pack")
    return st


def nm_spense_pack_workspace_size(o: int, k: int, axis: int, n_sparse: int) -> int:
    return int(lib().nm_spense_pack_workspace_size(o, k, axis, n_sparse))


def nm_spense_outsplit_gemm(x, ws_values, ws_meta, o_s, wd, o_d, y, accumulate=0, workspace=None, stream=None, *,
                            t=None, k=None, ldx=None, ldwd=None, ldy=None, workspace_bytes=None, check=True):
    t = x.shape[0] if t is None else t
    k = x.shape[1] if k is None else k
    wsb = (workspace.numel() * workspace.element_size() if workspace is not None else 0) \
        if workspace_bytes is None else workspace_bytes
    st = lib().nm_spense_outsplit_gemm(_ptr(x), t, k, _ld(x) if ldx is None else ldx, _ptr(ws_values),
                                       _ptr(ws_meta), o_s, _ptr(wd),
                                       (_ld(wd) if wd is not None else 0) if ldwd is None else ldwd, o_d, _ptr(y),
                                       _ld(y) if ldy is None else ldy, accumulate, _ptr(workspace), wsb,
                                       _stream(stream))
    if check:
        _check(st, "nm_spense_outsplit_gemm")
    return st


def nm_spense_outsplit_workspace_size(t: int, k: int, o_s: int, o_d: int) -> int:
    return int(lib().nm_spense_outsplit_workspace_size(t, k, o_s, o_d))


def nm_hybrid_gemm(x, sparse_cols, k_s, dense_cols, k_d, ws_values, ws_meta, fmt, wd, o, y, accumulate=0,
                   stream=None, *, t=None, ldx=None, ldwd=None, ldy=None, workspace=None, workspace_bytes=None,
                   route=0, taken=None, check=True):
    """taken: optional ctypes.c_uint32 that receives the NM_TAKEN_* report."""
    t = x.shape[0] if t is None else t
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    st = lib().nm_hybrid_gemm(_ptr(x), t, _ld(x) if ldx is None else ldx, _ptr(sparse_cols), k_s,
                              _ptr(dense_cols), k_d, _ptr(ws_values), _ptr(ws_meta), fmt, _ptr(wd),
                              _ld(wd) if ldwd is None else ldwd, o, _ptr(y), _ld(y) if ldy is None else ldy,
                              accumulate, _ptr(workspace), workspace_bytes, route,
                              ctypes.addressof(taken) if taken is not None else None, _stream(stream))
    if check:
        _check(st, "nm_hybrid_gemm")
    return st
