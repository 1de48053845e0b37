"""Pins of the fp64 oracle against things other than itself (CPU only).

Source: "Placement Is Free, Composition Is Not: The Latin Square as a Provably-Balanced
Construction for Heterogeneous Sequence-Mixer Stacks": Table 1 (full, sliding, differential),
sec. 8 (causal safety audit with a positive control).

Each pin is chosen so that a plausible mistake in the oracle fails at least one of them:
  * decimal brute force (50 digits, matrix form)      -> any indexing / mask / split slip
  * torch fp64 scaled_dot_product_attention            -> scale, causal convention
  * closed forms (row 0, L = 2 logistic, q = 0 means)  -> scale, normalisation, window edge
  * one zero half of q for differential                -> which half is which, sign of lambda
  * invariants (V = 1, W >= L, W = 1, shift of k, head permutation, row subsets)
  * causal and window audits, with planted faults that must be caught
"""
import math
import zlib

import numpy as np
import pytest
import torch

from bruteforce import attention_decimal

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force (decimal)

BRUTE_CASES = []
for L in (1, 2, 5, 12):
    for d in (2, 4, 8):
        BRUTE_CASES.append(("full", L, d, 0, 0.0))
        for W in sorted({1, 2, 3, L, L + 5}):
            BRUTE_CASES.append(("sliding", L, d, W, 0.0))
        for lam in (0.0, 0.8, -0.3):
            BRUTE_CASES.append(("differential", L, d, 0, lam))


@pytest.mark.parametrize("variant,L,d,W,lam", BRUTE_CASES)
def test_oracle_matches_decimal_bruteforce(oracle_mod, variant, L, d, W, lam):
    seed = zlib.crc32(repr((variant, L, d, W, lam)).encode())
    q, k, v = (_rand(seed + t, 1, 2, L, d) for t in range(3))
    got = oracle_mod.prefill(q, k, v, variant, W, lam)
    for h in range(2):
        ref = np.array(attention_decimal(q[0, h], k[0, h], v[0, h], variant, W, lam))
        np.testing.assert_allclose(got[0, h], ref, rtol=0, atol=1e-13)


# ------------------------------------------------------- library routine: torch SDPA fp64

def _sdpa(q, k, v, scale, mask=None, causal=False):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], attn_mask=m, is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("L,d", [(37, 16), (130, 64), (64, 128)])
def test_full_matches_torch_sdpa_causal(oracle_mod, L, d):
    q, k, v = (_rand(10 + t, 2, 3, L, d) for t in range(3))
    got = oracle_mod.prefill(q, k, v, "full")
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(d), causal=True)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,d,W", [(50, 16, 7), (130, 64, 64), (90, 32, 1), (40, 8, 40)])
def test_sliding_matches_torch_sdpa_band(oracle_mod, L, d, W):
    q, k, v = (_rand(20 + t, 1, 2, L, d) for t in range(3))
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    band = (j <= i) & (i - j < W)
    got = oracle_mod.prefill(q, k, v, "sliding", W)
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(d), mask=band)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,d,lam", [(45, 16, 0.8), (130, 128, -0.3), (33, 64, 0.0)])
def test_differential_matches_two_torch_sdpa_maps(oracle_mod, L, d, lam):
    q, k, v = (_rand(30 + t, 1, 2, L, d) for t in range(3))
    h = d // 2
    s = 1.0 / math.sqrt(h)
    ref = (_sdpa(q[..., :h], k[..., :h], v, s, causal=True)
           - lam * _sdpa(q[..., h:], k[..., h:], v, s, causal=True))
    got = oracle_mod.prefill(q, k, v, "differential", 0, lam)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 3, 0.0),
                                           ("differential", 0, 0.8),
                                           ("differential", 0, -0.3)])
def test_row0_is_v0(oracle_mod, variant, W, lam):
    q, k, v = (_rand(40 + t, 1, 2, 9, 8) for t in range(3))
    got = oracle_mod.prefill(q, k, v, variant, W, lam)
    factor = (1.0 - lam) if variant == "differential" else 1.0
    np.testing.assert_allclose(got[:, :, 0], factor * v[:, :, 0], rtol=0, atol=1e-15)


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("d", [4, 64, 128])
def test_two_tokens_logistic_full(oracle_mod, d):
    q, k, v = (_rand(50 + t, 1, 1, 2, d) for t in range(3))
    got = oracle_mod.prefill(q, k, v, "full")[0, 0, 1]
    s = 1.0 / math.sqrt(d)
    g = _sigmoid(s * float(q[0, 0, 1] @ (k[0, 0, 1] - k[0, 0, 0])))
    ref = v[0, 0, 0] + g * (v[0, 0, 1] - v[0, 0, 0])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("d,lam", [(4, 0.8), (128, 0.8), (64, -0.3)])
def test_two_tokens_logistic_differential(oracle_mod, d, lam):
    q, k, v = (_rand(60 + t, 1, 1, 2, d) for t in range(3))
    h = d // 2
    s = 1.0 / math.sqrt(h)  # 1/8 at d = 128
    qi, dk = q[0, 0, 1], k[0, 0, 1] - k[0, 0, 0]
    g1 = _sigmoid(s * float(qi[:h] @ dk[:h]))
    g2 = _sigmoid(s * float(qi[h:] @ dk[h:]))
    v0, v1 = v[0, 0, 0], v[0, 0, 1]
    ref = (1.0 - lam) * v0 + (g1 - lam * g2) * (v1 - v0)
    got = oracle_mod.prefill(q, k, v, "differential", 0, lam)[0, 0, 1]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_zero_queries_give_prefix_and_window_means(oracle_mod):
    L, d, W = 70, 16, 9
    k, v = _rand(70, 1, 2, L, d), _rand(71, 1, 2, L, d)
    q = np.zeros_like(k)
    prefix = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    np.testing.assert_allclose(oracle_mod.prefill(q, k, v, "full"), prefix, rtol=0,
                               atol=1e-14)
    csum = np.concatenate([np.zeros((1, 2, 1, d)), np.cumsum(v, axis=2)], axis=2)
    lo = np.maximum(0, np.arange(L) - W + 1)
    hi = np.arange(L) + 1
    trailing = (csum[:, :, hi] - csum[:, :, lo]) / (hi - lo)[None, None, :, None]
    np.testing.assert_allclose(oracle_mod.prefill(q, k, v, "sliding", W), trailing, rtol=0,
                               atol=1e-13)
    np.testing.assert_allclose(oracle_mod.prefill(q, k, v, "differential", 0, 0.8),
                               0.2 * prefix, rtol=0, atol=1e-14)


@pytest.mark.parametrize("zero_half", [0, 1])
def test_differential_one_zero_half(oracle_mod, zero_half):
    """With one half of q zero, that map is uniform (a prefix mean) and the other is plain
    half-width attention: pins which half is map 1, the sign of lambda and the 1/sqrt(d/2)
    scale."""
    L, d, lam = 50, 32, 0.8
    q, k, v = (_rand(80 + t, 1, 1, L, d) for t in range(3))
    h = d // 2
    if zero_half == 0:
        q[..., :h] = 0.0
    else:
        q[..., h:] = 0.0
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    half = slice(h, d) if zero_half == 0 else slice(0, h)
    att = oracle_mod.attention_general(q[0, 0, :, half], k[0, 0, :, half], v[0, 0],
                                       1.0 / math.sqrt(h))
    ref = (prefix - lam * att) if zero_half == 0 else (att - lam * prefix)
    got = oracle_mod.prefill(q, k, v, "differential", 0, lam)[0, 0]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


# ------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("variant,W,lam,expect", [("full", 0, 0.0, 1.0),
                                                  ("sliding", 5, 0.0, 1.0),
                                                  ("differential", 0, 0.8, 0.2),
                                                  ("differential", 0, -0.3, 1.3)])
def test_rows_sum_to_one(oracle_mod, variant, W, lam, expect):
    q, k = _rand(90, 1, 2, 40, 16), _rand(91, 1, 2, 40, 16)
    v = np.ones_like(q)
    got = oracle_mod.prefill(q, k, v, variant, W, lam)
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("W", [57, 58, 1000])
def test_window_at_least_L_equals_full(oracle_mod, W):
    q, k, v = (_rand(100 + t, 1, 2, 57, 16) for t in range(3))
    a = oracle_mod.prefill(q, k, v, "sliding", W)
    b = oracle_mod.prefill(q, k, v, "full")
    assert np.array_equal(a, b)


def test_window_one_is_v(oracle_mod):
    q, k, v = (_rand(110 + t, 2, 2, 33, 16) for t in range(3))
    assert np.array_equal(oracle_mod.prefill(q, k, v, "sliding", 1), v)


@pytest.mark.parametrize("lam", [0.8, 0.0, -0.3])
def test_differential_equal_halves(oracle_mod, lam):
    L, d = 60, 32
    h = d // 2
    q, k, v = (_rand(120 + t, 1, 1, L, d) for t in range(3))
    q[..., h:] = q[..., :h]
    k[..., h:] = k[..., :h]
    got = oracle_mod.prefill(q, k, v, "differential", 0, lam)[0, 0]
    ref = (1.0 - lam) * oracle_mod.attention_general(q[0, 0, :, :h], k[0, 0, :, :h], v[0, 0],
                                                     1.0 / math.sqrt(h))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 6, 0.0),
                                           ("differential", 0, 0.8)])
def test_constant_key_shift_is_invisible(oracle_mod, variant, W, lam):
    q, k, v = (_rand(130 + t, 1, 2, 40, 16) for t in range(3))
    u = _rand(133, 16)
    a = oracle_mod.prefill(q, k, v, variant, W, lam)
    b = oracle_mod.prefill(q, k + u, v, variant, W, lam)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_head_and_batch_permutation(oracle_mod):
    q, k, v = (_rand(140 + t, 2, 3, 30, 16) for t in range(3))
    perm_b, perm_h = [1, 0], [2, 0, 1]
    for variant, W, lam in (("full", 0, 0.0), ("sliding", 4, 0.0), ("differential", 0, 0.5)):
        a = oracle_mod.prefill(q, k, v, variant, W, lam)
        pq, pk, pv = (x[perm_b][:, perm_h] for x in (q, k, v))
        b = oracle_mod.prefill(pq, pk, pv, variant, W, lam)
        assert np.array_equal(a[perm_b][:, perm_h], b)


def test_row_subset_equals_full_rows(oracle_mod):
    q, k, v = (_rand(150 + t, 1, 2, 100, 16) for t in range(3))
    rows = [99, 0, 50, 7, 7]
    for variant, W, lam in (("full", 0, 0.0), ("sliding", 10, 0.0), ("differential", 0, 0.8)):
        a = oracle_mod.prefill(q, k, v, variant, W, lam)
        b = oracle_mod.prefill_rows(q, k, v, variant, W, lam, rows)
        assert np.array_equal(a[:, :, rows], b)


def test_thread_count_does_not_change_bits(oracle_mod):
    q, k, v = (_rand(160 + t, 1, 2, 200, 16) for t in range(3))
    a = oracle_mod.prefill(q, k, v, "differential", 0, 0.8, threads=1)
    b = oracle_mod.prefill(q, k, v, "differential", 0, 0.8, threads=0)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments(oracle_mod):
    q = np.zeros((1, 1, 4, 3))
    with pytest.raises(ValueError):
        oracle_mod.prefill(q, q, q, "differential", 0, 0.8)   # odd d
    q = np.zeros((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle_mod.prefill(q, q, q, "sliding", 0)             # window < 1
    with pytest.raises(ValueError):
        oracle_mod.prefill_rows(q, q, q, "full", rows=[4])    # row out of range


# ------------------------------------------------ causal audit (sec. 8), with a positive control

def _future_leak_rows(oracle_mod, variant, W, lam, plant, L=48, d=8, t=20):
    """Perturb every input at positions > t; return whether rows <= t changed."""
    q, k, v = (_rand(170 + s, 1, 2, L, d) for s in range(3))
    a = oracle_mod.prefill_rows(q, k, v, variant, W, lam, plant=plant)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, :, t + 1:] += _rand(175, *x[:, :, t + 1:].shape)
    b = oracle_mod.prefill_rows(q2, k2, v2, variant, W, lam, plant=plant)
    return not np.array_equal(a[:, :, :t + 1], b[:, :, :t + 1])


def _window_leak_rows(oracle_mod, W, plant, L=48, d=8, i=30):
    """Perturb keys and values at positions <= i - W; return whether row i changed."""
    q, k, v = (_rand(180 + s, 1, 2, L, d) for s in range(3))
    a = oracle_mod.prefill_rows(q, k, v, "sliding", W, rows=[i], plant=plant)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :i - W + 1] += 1.5
    v2[:, :, :i - W + 1] -= 2.0
    b = oracle_mod.prefill_rows(q, k2, v2, "sliding", W, rows=[i], plant=plant)
    return not np.array_equal(a, b)


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 5, 0.0),
                                           ("differential", 0, 0.8)])
def test_causal_audit_negative_control(oracle_mod, variant, W, lam):
    assert not _future_leak_rows(oracle_mod, variant, W, lam, plant=0)


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 5, 0.0),
                                           ("differential", 0, 0.8)])
def test_causal_audit_positive_control(oracle_mod, variant, W, lam):
    # plant 1 lets one future key through; the audit must notice.
    assert _future_leak_rows(oracle_mod, variant, W, lam, plant=1)


@pytest.mark.parametrize("W", [1, 5, 17])
def test_window_audit_controls(oracle_mod, W):
    assert not _window_leak_rows(oracle_mod, W, plant=0)
    assert _window_leak_rows(oracle_mod, W, plant=2)
