"""Seeded synthetic inputs shared by the tests, the oracle side and the benchmark.

This module only draws random numbers and lays them out in the storage formats the
library consumes (bf16 bit patterns, fp8-e4m3 bytes with per-row scales).  It holds
none of the sparsification arithmetic: no selection, no compression, no lowering,
no product.  Both the CPU oracle and the GPU path receive byte-identical arrays from
here.

Shapes and distributions follow the workloads of the sparse-linear-layer papers:
8B-class transformer shapes (hidden 4096, intermediate 14336, kv 1024), weights
N(0, 0.02) (read as standard deviation 0.02), activations N(0, 1) or Student-t with
4 degrees of freedom (heavy-tailed post-SiLU activations, scaled by 0.5 for the
down-projection workload).
"""
from __future__ import annotations

import hashlib

import numpy as np

__all__ = [
    "bf16_bits_from_f32", "f32_from_bf16_bits", "normal_bf16", "student_t_bf16",
    "fp8_e4m3_quantize_rows", "sha256", "layer_2of4_small", "mlp_down_8of16",
    "slide_6of8_layer", "hybrid_up_layer", "transformer_layer", "device_normal_bf16",
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits_from_f32(x)


def student_t_bf16(rng: np.random.Generator, shape, nu: float = 4.0, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_t(nu, size=shape).astype(np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_bits_from_f32(x)


def fp8_e4m3_quantize_rows(w_bits: np.ndarray):
    """Storage format of the fp8 weight variant: per-output-row scale s = max|w| / 448
    (fp32; 1 for an all-zero row) and codes q = e4m3fn(w / s), round to nearest even.

    This produces an input weight format; the library and the oracle only decode it.
    The rounding is done by torch's CPU fp8 conversion.
    """
    import torch

    w = f32_from_bf16_bits(w_bits)
    amax = np.abs(w).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    q = torch.from_numpy((w / s[:, None]).astype(np.float32)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), s


def device_normal_bf16(torch, shape, seed: int, std: float = 1.0):
    """N(0, std) drawn on the GPU from a seeded generator and rounded to bf16 (nearest
    even), returned as a device int16 tensor of bf16 bit patterns.  For inputs too large
    to draw on the host; tests copy the rows they check back to the host."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if std != 1.0:
        x *= std
    return x.to(torch.bfloat16).view(torch.int16)


def sha256(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------------------
# Workload recipes.  Each returns a dict of uint16 bf16-bit arrays (row-major, K fastest).
# Weights are drawn first, then activations, from one generator per workload.
# --------------------------------------------------------------------------------------

def layer_2of4_small(seed: int = 0):
    """Single 2:4 activation-sparse linear layer: X 64x512 ~ N(0,1), W 512x512 ~ N(0,0.02).
    One generator, X drawn first, then W."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (64, 512), 1.0)
    w = normal_bf16(rng, (512, 512), 0.02)
    return {"x": x, "w": w, "n": 2, "m": 4}


def mlp_down_8of16(t_max: int = 8192, seed: int = 2, k: int = 14336, o: int = 4096):
    """8:16 activation sparsity on an MLP down-projection: W o x k ~ N(0,0.02);
    X t_max x k Student-t(4) * 0.5.  Smaller token counts use the first rows of X."""
    rng = np.random.default_rng(seed)
    w = normal_bf16(rng, (o, k), 0.02)
    x = student_t_bf16(rng, (t_max, k), 4.0, 0.5)
    return {"x": x, "w": w, "n": 8, "m": 16}


def slide_6of8_layer(t_max: int = 4096, seed: int = 3, k: int = 4096, o: int = 4096):
    """Dense W o x k ~ N(0,0.02) (to be magnitude-pruned 6:8 by the library) and
    X t_max x k ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = normal_bf16(rng, (o, k), 0.02)
    x = normal_bf16(rng, (t_max, k), 1.0)
    return {"x": x, "w": w, "ns": 4}


def hybrid_up_layer(t_max: int = 2048, seed: int = 4, k: int = 4096, o: int = 14336, dense_frac: float = 0.25):
    """W o x k ~ N(0,0.02) for the hybrid dense + 2:4 split (25% of K columns dense),
    X t_max x k ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = normal_bf16(rng, (o, k), 0.02)
    x = normal_bf16(rng, (t_max, k), 1.0)
    return {"x": x, "w": w, "k_dense": int(round(k * dense_frac))}


TRANSFORMER_SHAPES = {
    # name: (out_features, in_features, input stream)
    "q": (4096, 4096, "attn_in"), "k": (1024, 4096, "attn_in"), "v": (1024, 4096, "attn_in"),
    "o": (4096, 4096, "o_in"), "gate": (14336, 4096, "mlp_in"), "up": (14336, 4096, "mlp_in"),
    "down": (4096, 14336, "down_in"),
}


def transformer_layer(t_max: int = 8192, seed: int = 5, names=None, with_fp8: bool = False):
    """One 8B-shaped transformer layer: the seven linears with bf16 weights ~ N(0,0.02)
    (drawn q, k, v, o, gate, up, down), then four Student-t(4) activation streams
    (attn_in, o_in, mlp_in, down_in) of t_max rows each.  `names` restricts which
    weights are kept (all are still drawn, so the streams do not depend on it)."""
    rng = np.random.default_rng(seed)
    out = {"w": {}, "x": {}, "w8": {}, "s8": {}}
    for nm, (o, k, _) in TRANSFORMER_SHAPES.items():
        w = normal_bf16(rng, (o, k), 0.02)
        if names is None or nm in names:
            out["w"][nm] = w
            if with_fp8:
                out["w8"][nm], out["s8"][nm] = fp8_e4m3_quantize_rows(w)
    streams = {"attn_in": 4096, "o_in": 4096, "mlp_in": 4096, "down_in": 14336}
    for st, k in streams.items():
        x = student_t_bf16(rng, (t_max, k), 4.0, 1.0)
        if names is None or any(TRANSFORMER_SHAPES[nm][2] == st for nm in names):
            out["x"][st] = x
    return out
