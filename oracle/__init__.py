"""Oracle: a plain, slow, obviously correct CPU reference for the mixer hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the HIP library
and its Python binding) never imports, links or runs anything here, and this package never
imports the product.

Contents
  * ``prefill`` / ``prefill_rows`` / ``attention_general``: ctypes wrappers of the fp64 C
    loops in ``oracle.c`` (the attention definition written out per query row).
  * ``prefill_rows_gqa``: the same layer with key/value heads shared by groups of query
    heads (Table 2, sec. 4.1).
  * ``latin``: the Latin-square schedule definitions in plain Python.

Source: "Placement Is Free, Composition Is Not: The Latin Square as a Provably-Balanced
Construction for Heterogeneous Sequence-Mixer Stacks" (Table 1, sec. 3.2, sec. 4.1 Table 2,
sec. 8, Table 7).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import latin  # noqa: F401  (re-exported)

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FULL, SLIDING, DIFFERENTIAL = 0, 1, 2
VARIANTS = {"full": FULL, "sliding": SLIDING, "differential": DIFFERENTIAL}

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (strict IEEE: no fast-math, no
    contraction of a*b+c into fused multiply-adds)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = ctypes.CDLL(LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    cl, ci, cd = ctypes.c_long, ctypes.c_int, ctypes.c_double
    lib.oracle_prefill_rows.argtypes = [dp, dp, dp, ci, cl, cd, cl, cl, cl, cl, lp, cl, dp, ci,
                                        ci]
    lib.oracle_prefill_rows.restype = ci
    lib.oracle_attention_general.argtypes = [dp, dp, dp, cl, cl, cl, cd, cl, dp, ci]
    lib.oracle_attention_general.restype = ci
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ci
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def prefill_rows(q, k, v, variant, window: int = 0, lam: float = 0.0, rows=None,
                 threads: int = 0, plant: int = 0) -> np.ndarray:
    """One mixer layer on [B, H, L, d] inputs (any real dtype, widened to float64).

    ``variant`` is 0/1/2 or "full"/"sliding"/"differential". ``rows`` (optional) lists the
    query rows to compute for every (b, h); the result is then [B, H, len(rows), d].
    ``plant`` is the positive-control hook of the causal audit and must stay 0 elsewhere.
    """
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B, H, L, d] shape: {q.shape} {k.shape} "
                         f"{v.shape}")
    B, H, L, d = q.shape
    if rows is None:
        rows_arr = None
        n = L
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
    out = np.empty((B, H, n, d), dtype=np.float64)
    rc = _load().oracle_prefill_rows(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        int(variant), int(window), float(lam), B, H, L, d,
        None if rows_arr is None else _ptr(rows_arr, ctypes.c_long), n,
        _ptr(out, ctypes.c_double), int(threads), int(plant))
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (variant={variant}, window={window}, "
                         f"shape={q.shape}, rows={rows is not None})")
    return out


def prefill_rows_gqa(q, k, v, variant, window: int = 0, lam: float = 0.0, rows=None,
                     threads: int = 0) -> np.ndarray:
    """One mixer layer with grouped key/value heads: q [B, H, L, d], k and v [B, Hkv, L, d]
    with Hkv dividing H. The model the paper builds uses 16 heads over 4 KV heads (Table 2,
    sec. 4.1); query head h attends with key/value head h // (H // Hkv), and is otherwise the
    layer ``prefill_rows`` computes. Written out as exactly that: each key/value head repeated
    for the H // Hkv query heads that share it, then ``prefill_rows``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError(f"q [B, H, L, d], k and v [B, Hkv, L, d]: {q.shape} {k.shape} "
                         f"{v.shape}")
    B, H, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"k and v must be [B, Hkv, L, d] with Hkv dividing H: {k.shape}")
    g = H // Hkv
    return prefill_rows(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), variant, window,
                        lam, rows, threads)


def prefill(q, k, v, variant, window: int = 0, lam: float = 0.0, threads: int = 0):
    """Every row of one mixer layer; see ``prefill_rows``."""
    return prefill_rows(q, k, v, variant, window, lam, None, threads)


def attention_general(q, k, v, scale: float, window: int = 0, threads: int = 0):
    """Single-head causal softmax attention with independent widths: q, k [L, dqk],
    v [L, dv], explicit scale; ``window`` >= 1 adds the sliding window."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, dqk = q.shape
    dv = v.shape[1]
    if k.shape != (L, dqk) or v.shape[0] != L:
        raise ValueError("shape mismatch")
    out = np.empty((L, dv), dtype=np.float64)
    rc = _load().oracle_attention_general(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        L, dqk, dv, float(scale), int(window), _ptr(out, ctypes.c_double), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out

