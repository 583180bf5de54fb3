"""Helpers shared by the GPU tests: host<->device copies of bit arrays, the GEMM tolerance
check (relative Frobenius <= 1e-3 and |err| <= 1e-2 * (|A|.|B|) + 1e-4 against the oracle's
fp32-accumulated product), and the whole-output checks of full-size products: one row of
every band of output rows against the oracle, no unwritten (NaN pre-filled) element
anywhere, and random projections of the whole output."""
import numpy as np

import oracle as O

REL_FRO = 1e-3
ELT_REL = 1e-2
ELT_ABS = 1e-4


def dev(a, ld=None):
    """numpy array -> CUDA tensor with the same bytes; optional padded leading dim."""
    import torch

    a = np.ascontiguousarray(a)
    if ld is not None and ld != a.shape[1]:
        pad = np.zeros((a.shape[0], ld), dtype=a.dtype)
        pad[:, :a.shape[1]] = a
        a = pad
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype)
    t = torch.from_numpy(a.view(view) if view is not None else a)
    return t.cuda()


def host(t, dtype):
    return t.cpu().numpy().view(dtype)


def empty(shape, dtype, fill=None):
    import torch

    tdt = {np.uint16: torch.int16, np.uint8: torch.uint8, np.uint32: torch.int32, np.float32: torch.float32,
           np.int32: torch.int32}[dtype]
    t = torch.empty(shape, dtype=tdt, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def check_gemm(y, y_ref, a_bits, b_bits, rows=None, label=""):
    """y: GPU fp32 [T][O]; y_ref: oracle fp64; a_bits [T][K], b_bits [O][K] are the operands
    actually contracted (for the |A|.|B| bound); b may instead be fp64 values (fp8 weights
    dequantised with their scales).  rows: optional subset of T."""
    y = np.asarray(y, dtype=np.float64)
    if rows is not None:
        y = y[rows]
    a = np.abs(O.bf16_to_f64(a_bits if rows is None else a_bits[rows]))
    b = np.abs(O.bf16_to_f64(b_bits)) if b_bits.dtype == np.uint16 else np.abs(np.asarray(b_bits, np.float64))
    bound = a @ b.T
    err = np.abs(y - y_ref)
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    worst = (err - ELT_REL * bound - ELT_ABS).max() if err.size else -1
    assert rel <= REL_FRO, f"{label} relative Frobenius error {rel:.3e}"
    assert worst <= 0, f"{label} per-element bound exceeded by {worst:.3e}"
    return rel


def sample_rows(t, count=48, seed=0):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(t, size=min(count, t), replace=False).tolist())
    r.update({0, t - 1})
    return np.array(sorted(r))


def check_gemm_vals(y, y_ref, a_vals, b_vals, label=""):
    """check_gemm with both operands given as fp64 values (e.g. dequantized fp8 codes)."""
    y = np.asarray(y, dtype=np.float64)
    bound = np.abs(np.asarray(a_vals, np.float64)) @ np.abs(np.asarray(b_vals, np.float64)).T
    err = np.abs(y - y_ref)
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    worst = (err - ELT_REL * bound - ELT_ABS).max() if err.size else -1
    assert rel <= REL_FRO, f"{label} relative Frobenius error {rel:.3e}"
    assert worst <= 0, f"{label} per-element bound exceeded by {worst:.3e}"
    return rel


def band_rows(t, band=128, seed=0):
    """One random row from every band of `band` consecutive output rows (so every tile of
    rows of that height has a checked row), plus the first and the last row."""
    rng = np.random.default_rng(seed)
    r = {0, t - 1}
    for b0 in range(0, t, band):
        r.add(int(rng.integers(b0, min(t, b0 + band))))
    return np.array(sorted(r))


def check_all_written(y_dev, label=""):
    """The output was pre-filled with NaN: every element must have been written with a
    finite value (checked on the device, over the whole output)."""
    import torch

    bad = int((~torch.isfinite(y_dev)).sum().item())
    assert bad == 0, f"{label}: {bad} output elements unwritten or not finite"


def check_projection(y, a_vals, b_vals, label="", nproj=8, seed=0):
    """Whole-output check through random projections: (A . B^T) . R = A . (B^T . R) for a
    Gaussian R [O][nproj].  A wrong or misplaced tile anywhere in y changes its projections
    by about its share of the output's norm, far above the 1e-3 relative bound.
    a_vals [T][K] and b_vals [O][K] are the operands contracted (fp64 values), y the
    output [T][O] (host)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.random.default_rng(seed).standard_normal((y.shape[1], nproj))
    got = y @ r
    ref = np.asarray(a_vals, np.float64) @ (np.asarray(b_vals, np.float64).T @ r)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_FRO, f"{label}: projection relative error {rel:.3e}"
    return rel
