"""Seeded synthetic inputs for the ConvRot low-bit linear path.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It holds no arithmetic of the method itself (no rotation, no
quantization, no integer GEMM, no epilogue): it only draws random tensors
with the shapes and value distributions of the workloads and rounds them
once to bfloat16, which is the input format of the path.

Shapes come from the per-family shape table of the "Qwen-Image-Edit-2511-W4A8-ConvRot"
model card (per-layer error section: [3072,3072], [3072,12288], [12288,3072],
[18432,3072]); the mixed recipe (which layers are INT4 and which INT8) from the
"Qwen-Image-Edit-2511 — INT4 tensorwise W4A4 (+ConvRot, mixed int8 fallback)"
page, intro. No dataset, prompt set or checkpoint is used: every tensor here
stands in for real MMDiT activations and weights.

Recipe (all tensors row-major; weights are [N, K] = [out, in]):
  * generator: numpy default_rng(SeedSequence([config_id, tensor_id]))
  * activations ~ N(0, 1) in float64, optional outlier channels (a fixed
    number of columns chosen without replacement and multiplied by a factor
    in float32 before rounding), then float32, then one RNE rounding to bf16
  * post-GELU activations: GELU(z) = z * Phi(z) with the exact erf, z ~ N(0,1)
  * weights ~ N(0, 0.02)
  * low-rank split (W = L1 @ L2 + R): float64 SVD of the bf16 weight, L1 =
    U_r * sigma_r and L2 = V_r^T rounded to bf16, R = W - L1 @ L2 computed in
    float64 from the rounded factors and rounded to bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits_from_f32", "f32_from_bf16_bits", "rng_for",
    "activation", "gelu_activation", "weight", "lowrank_split",
    "CONFIGS", "LinearSpec",
]


# --------------------------------------------------------------------------
# bf16 helpers (input format only)
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-half-to-even); return the
    16-bit patterns as uint16. Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    b = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return ((b + bias) >> np.uint64(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(tensor_id)]))


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def activation(config_id: int, tensor_id: int, M: int, K: int,
               n_outliers: int = 0, outlier_scale: float = 1.0) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1) with `n_outliers` columns scaled by
    `outlier_scale` (multiplied in float32 before the single bf16 rounding)."""
    g = rng_for(config_id, tensor_id)
    x = g.standard_normal((M, K)).astype(np.float32)
    if n_outliers > 0:
        cols = g.choice(K, size=n_outliers, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return bf16_bits_from_f32(x)


def gelu_activation(config_id: int, tensor_id: int, M: int, K: int) -> np.ndarray:
    """bf16 bits [M, K] of GELU(z), z ~ N(0,1), exact-erf GELU in float64."""
    g = rng_for(config_id, tensor_id)
    from scipy.special import erf
    z = g.standard_normal((M, K))
    phi = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    return bf16_bits_from_f32((z * phi).astype(np.float32))


def weight(config_id: int, tensor_id: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """bf16 bits [N, K] ~ N(0, std)."""
    g = rng_for(config_id, tensor_id)
    return bf16_bits_from_f32((g.standard_normal((N, K)) * std).astype(np.float32))


def lowrank_split(w_bits: np.ndarray, rank: int):
    """Low-rank plus residual split of a bf16 weight for the low-rank-corrected
    (SVD-style) workload: returns (L1 [N, rank], L2 [rank, K], R [N, K]) as bf16
    bits with W ~= L1 @ L2 + R. This is input synthesis: the offline split is
    not part of the timed path."""
    w = f32_from_bf16_bits(w_bits).astype(np.float64)
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    l1 = bf16_bits_from_f32((u[:, :rank] * s[:rank]).astype(np.float32))
    l2 = bf16_bits_from_f32(vt[:rank, :].astype(np.float32))
    lr = f32_from_bf16_bits(l1).astype(np.float64) @ f32_from_bf16_bits(l2).astype(np.float64)
    r = bf16_bits_from_f32((w - lr).astype(np.float32))
    return l1, l2, r


# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------

@dataclass
class LinearSpec:
    """One quantized linear of a workload.

    fmt: "w4a4" (INT4 x INT4, tensorwise), "int8" (INT8 x INT8, tensorwise),
         "w4a8" (asym uint4 g16 weights x per-token int8 activations),
         "w4a4_g64" (low-rank corrected, per-64-group scales),
         "a8w4" (W4A4-format weights, tensorwise, x per-token int8 activations)
    x_id: which activation tensor feeds it (layers that share an input share
          one rotate+quantize pass).
    chain: layers of one chain run in order; different chains are independent
           (the image and text token streams of an MMDiT block) and may run
           concurrently.
    phase: chains meet between phases: every layer of phase p runs after
           every layer of phase p - 1 of all chains (the joint attention of an
           MMDiT block reads the Q, K and V of both token streams, and each
           stream's output projection reads the attention's output).
    parts: for a layer that runs several linears of the same input as one
           call (their weights side by side along N), those linears; empty
           for an ordinary layer.
    """
    name: str
    fmt: str
    M: int
    N: int
    K: int
    x_id: str
    rot: int = 256
    unsigned_shift: float = 0.0
    rank: int = 0
    chain: str = ""
    phase: int = 0
    parts: tuple = ()


@dataclass
class Workload:
    config_id: int
    name: str
    linears: list = field(default_factory=list)
    # activation tensors: id -> (M, K, kind, n_outliers, outlier_scale)
    acts: dict = field(default_factory=dict)


def _c1():
    w = Workload(1, "tiny W4A4 tensorwise ConvRot linear 64x256x512")
    w.acts["x"] = (64, 512, "normal", 5, 20.0)
    w.linears.append(LinearSpec("proj", "w4a4", 64, 256, 512, "x"))
    return w


def _c2(M: int):
    w = Workload(2, f"MMDiT projection W4A4 tensorwise ConvRot {M}x3072x3072")
    w.acts["x"] = (M, 3072, "normal", 15, 30.0)
    w.linears.append(LinearSpec("proj", "w4a4", M, 3072, 3072, "x"))
    return w


def _c3():
    w = Workload(3, "W4A8 asym g16 linear 8192x12288x3072")
    w.acts["x"] = (8192, 3072, "normal", 0, 1.0)
    w.linears.append(LinearSpec("mlp_up", "w4a8", 8192, 12288, 3072, "x"))
    return w


def _c4(m_img: int = 8192, m_txt: int = 512, m_mod: int = 2):
    w = Workload(4, f"mixed MMDiT block {m_img} img + {m_txt} txt tokens, hidden 3072")
    for s, M in (("img", m_img), ("txt", m_txt)):
        w.acts[f"{s}_attn"] = (M, 3072, "normal", 0, 1.0)
        w.acts[f"{s}_attnout"] = (M, 3072, "normal", 0, 1.0)
        w.acts[f"{s}_mlp"] = (M, 3072, "normal", 0, 1.0)
        w.acts[f"{s}_gelu"] = (M, 12288, "gelu", 0, 1.0)
        w.linears += [
            LinearSpec(f"{s}_q", "w4a4", M, 3072, 3072, f"{s}_attn", chain=s),
            LinearSpec(f"{s}_k", "w4a4", M, 3072, 3072, f"{s}_attn", chain=s),
            LinearSpec(f"{s}_v", "int8", M, 3072, 3072, f"{s}_attn", chain=s),
            LinearSpec(f"{s}_out", "int8", M, 3072, 3072, f"{s}_attnout", chain=s, phase=1),
            LinearSpec(f"{s}_mlp_up", "w4a4", M, 12288, 3072, f"{s}_mlp", chain=s, phase=1),
            LinearSpec(f"{s}_mlp_down", "w4a4", M, 3072, 12288, f"{s}_gelu", chain=s, phase=1),
        ]
        w.acts[f"{s}_mod"] = (m_mod, 3072, "normal", 0, 1.0)
        w.linears.append(LinearSpec(f"{s}_mod", "int8", m_mod, 18432, 3072, f"{s}_mod", chain=s, phase=1))
    return w


def _c5(M: int = 8192):
    w = Workload(5, f"low-rank corrected W4A4 g64, split QKV + unsigned MLP down, {M} tokens")
    w.acts["x"] = (M, 3072, "normal", 0, 1.0)
    w.acts["gelu"] = (M, 12288, "gelu", 0, 1.0)
    w.linears.append(LinearSpec("qkv", "w4a4_g64", M, 9216, 3072, "x", rot=0, rank=32))
    w.linears.append(LinearSpec("mlp_down", "w4a4_g64", M, 3072, 12288, "gelu", rot=0,
                                unsigned_shift=0.171875, rank=32))
    return w


def _c2pair():
    """The MMDiT projection of C2 at both token counts in one step: image
    tokens (M = 4096, fp6 codes) and the small-token case (M = 32)."""
    w = Workload(2, "MMDiT projection W4A4 tensorwise ConvRot (4096 + 32)x3072x3072")
    for M in (4096, 32):
        w.acts[f"x{M}"] = (M, 3072, "normal", 15, 30.0)
        w.linears.append(LinearSpec(f"proj{M}", "w4a4", M, 3072, 3072, f"x{M}", chain=f"m{M}"))
    return w


def _c2a8():
    """The MMDiT projection of C2 on the 8-bit-activation branch: the same
    W4A4-format weights against per-token INT8 activations (M = 4096 and 32)."""
    w = Workload(2, "MMDiT projection, W4A4-format weights x per-token INT8 activations, (4096 + 32)x3072x3072")
    for M in (4096, 32):
        w.acts[f"x{M}"] = (M, 3072, "normal", 15, 30.0)
        w.linears.append(LinearSpec(f"proj{M}", "a8w4", M, 3072, 3072, f"x{M}"))
    return w


CONFIGS = {
    "c1": _c1,
    "c2_m32": lambda: _c2(32),
    "c2_m4096": lambda: _c2(4096),
    "c2": _c2pair,
    "c3": _c3,
    "c4": _c4,
    "c5": _c5,
    "c2a8": _c2a8,
}


# --------------------------------------------------------------------------
# per-workload tensors (shared by the full-size tests and the benchmark, so
# both draw exactly the same inputs)
# --------------------------------------------------------------------------

def act_bits(w: Workload, name: str, rows: int | None = None) -> np.ndarray:
    """bf16 bits of activation tensor `name` of workload `w`; `rows` draws
    only its first rows (the same values: the generator fills the tensor row
    by row; tensors with outlier columns are drawn whole and cut)."""
    M, K, kind, n_out, scale = w.acts[name]
    tid = 100 + sorted(w.acts).index(name)
    if rows is not None and n_out:
        return act_bits(w, name)[:rows]
    Mr = M if rows is None else min(M, rows)
    if kind == "gelu":
        return gelu_activation(w.config_id, tid, Mr, K)
    return activation(w.config_id, tid, Mr, K, n_out, scale)


def weight_bits(w: Workload, lin: LinearSpec, rows: int | None = None) -> np.ndarray:
    """bf16 bits [N, K] of the weight of linear `lin` of workload `w` (its
    first `rows` output channels when given: the same values)."""
    tid = 200 + [l.name for l in w.linears].index(lin.name)
    return weight(w.config_id, tid, lin.N if rows is None else min(lin.N, rows), lin.K)


def lowrank_bits(w: Workload, lin: LinearSpec):
    """(L1 [N, rank], L2 [rank, K], R [N, K]) bf16 bits of a low-rank-corrected
    linear: the rank-`lin.rank` split of its weight (see lowrank_split)."""
    return lowrank_split(weight_bits(w, lin), lin.rank)


__all__ += ["Workload", "act_bits", "weight_bits", "lowrank_bits"]
