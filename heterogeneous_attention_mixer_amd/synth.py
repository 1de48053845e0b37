"""Seeded synthetic inputs for the mixer layer (shared by tests, the benchmark and the smoke
check; holds none of the method's arithmetic).

Recipe: numpy PCG64 ``default_rng(seed)`` draws Q, then K, then V, each with
``standard_normal(shape, dtype=float32)`` (N(0, 1), the distribution of unit-variance
normalised activations). For bf16 workloads the float32 draws are rounded to bfloat16 with
round-to-nearest-even on the host; those exact bits go to the device and, widened, to the
CPU reference. fp32 workloads keep the float32 draws.

Shapes follow the paper's attention layer: 16 heads of head_dim 128 (Table 2, "Placement Is
Free, Composition Is Not", sec. 4.1) at the context lengths of its cost profile (Table 3:
2K, 8K, 32K).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class LayerInputs:
    """One layer's q, k, v. ``bits`` holds bfloat16 patterns (uint16) for bf16 workloads and
    is None for fp32 ones; ``f32`` holds the exact float32 values of what the device sees."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None
    k_bits: np.ndarray | None
    v_bits: np.ndarray | None
    dtype: str

    @property
    def shape(self):
        return self.q.shape


def make_qkv(seed: int, B: int, H: int, L: int, d: int, dtype: str = "bf16") -> LayerInputs:
    """Draw q, k, v of shape [B, H, L, d] (in that order) from ``default_rng(seed)``."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    shape = (B, H, L, d)
    draws = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if dtype == "f32":
        return LayerInputs(draws[0], draws[1], draws[2], None, None, None, "f32")
    bits = [round_to_bf16_bits(x) for x in draws]
    vals = [bf16_bits_to_f32(b) for b in bits]
    return LayerInputs(vals[0], vals[1], vals[2], bits[0], bits[1], bits[2], "bf16")


def make_qkv_gqa(seed: int, B: int, H: int, Hkv: int, L: int, d: int) -> LayerInputs:
    """Grouped key/value heads: q [B, H, L, d], then k and v [B, Hkv, L, d], drawn in that
    order from ``default_rng(seed)`` and rounded to bf16 as in ``make_qkv``."""
    rng = np.random.default_rng(seed)
    draws = [rng.standard_normal(shape, dtype=np.float32)
             for shape in ((B, H, L, d), (B, Hkv, L, d), (B, Hkv, L, d))]
    bits = [round_to_bf16_bits(x) for x in draws]
    vals = [bf16_bits_to_f32(b) for b in bits]
    return LayerInputs(vals[0], vals[1], vals[2], bits[0], bits[1], bits[2], "bf16")


# Named workloads (seed, variant, window, lambda, B, H, L, d, dtype).
def make_mfma_fragments(seed: int, nsets: int) -> np.ndarray:
    """Operand fragments for the matrix-core ceiling measurement: ``nsets`` sets of 8
    fragments x 64 lanes x 8 elements, standard normal draws from ``default_rng(seed)``
    rounded to bf16 bits (uint16), shape (nsets, 8, 64, 8). Same statistics as q, k, v."""
    rng = np.random.default_rng(seed)
    return round_to_bf16_bits(rng.standard_normal((nsets, 8, 64, 8), dtype=np.float32))


# The ceiling measurement as the bench runs it: 512 workgroups of 4 waves (two per SIMD),
# each wave 4 chains of `iters` matrix instructions, about 5 ms per launch at 2 PFLOP/s.
MFMA_CEILING = dict(blocks=512, iters=36864, nsets=64, seed=700)

WORKLOADS = {
    "full_fp32_L256_d64": dict(seed=1, variant="full", window=0, lam=0.0,
                               B=1, H=2, L=256, d=64, dtype="f32"),
    "sliding_W1024_L8192": dict(seed=2, variant="sliding", window=1024, lam=0.0,
                                B=1, H=16, L=8192, d=128, dtype="bf16"),
    "full_L2048": dict(seed=3, variant="full", window=0, lam=0.0,
                       B=1, H=16, L=2048, d=128, dtype="bf16"),
    "full_L8192": dict(seed=3, variant="full", window=0, lam=0.0,
                       B=1, H=16, L=8192, d=128, dtype="bf16"),
    "full_L32768": dict(seed=3, variant="full", window=0, lam=0.0,
                        B=1, H=16, L=32768, d=128, dtype="bf16"),
    "differential_L8192": dict(seed=4, variant="differential", window=0, lam=0.8,
                               B=1, H=16, L=8192, d=128, dtype="bf16"),
    "differential_L32768": dict(seed=4, variant="differential", window=0, lam=0.8,
                                B=1, H=16, L=32768, d=128, dtype="bf16"),
}

# The model's own attention shape (Table 2, sec. 4.1: 16 heads over 4 KV heads, head_dim
# 128) at 8K, each variant drawn from seed 600 + variant number.
GQA = dict(B=1, H=16, Hkv=4, L=8192, d=128, window=1024, lam=0.8, seed0=600)

# The 3x3 Latin stack: base row [full, sliding, differential], window 1024, lambda 0.8,
# B=1, H=16, L=8192, d=128, bf16, layer l drawn from seed 500 + l.
LATIN_STACK = dict(base=("full", "sliding", "differential"), window=1024, lam=0.8,
                   B=1, H=16, L=8192, d=128, seed0=500)
