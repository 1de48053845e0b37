"""Pins of the oracle's grouped key/value heads (``prefill_rows_gqa``).

Grouped heads are the attention shape of the model in "Placement Is Free, Composition Is
Not" (Table 2, sec. 4.1: 16 heads over 4 KV heads): query head h attends with key/value head
h // (H // Hkv). Pinned against the 50-digit brute force, which indexes the shared key/value
head directly (no repetition), on tiny inputs; and against the plain layer for Hkv = H.
"""
import numpy as np
import pytest

from bruteforce import attention_decimal


def _inputs(seed, B, H, Hkv, L, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    return q, k, v


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 3, 0.0),
                                           ("differential", 0, 0.7)])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (4, 1), (6, 3)])
def test_gqa_matches_decimal_bruteforce(oracle_mod, variant, W, lam, H, Hkv):
    B, L, d = 2, 5, 4
    q, k, v = _inputs(100 + H + Hkv, B, H, Hkv, L, d)
    got = oracle_mod.prefill_rows_gqa(q, k, v, variant, W, lam)
    g = H // Hkv
    for b in range(B):
        for h in range(H):
            want = attention_decimal(q[b, h], k[b, h // g], v[b, h // g], variant, W, lam)
            np.testing.assert_allclose(got[b, h], np.asarray(want, dtype=np.float64),
                                       rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", ["full", "sliding", "differential"])
def test_gqa_with_one_head_per_group_is_the_plain_layer(oracle_mod, variant):
    q, k, v = _inputs(7, 1, 3, 3, 33, 8)
    a = oracle_mod.prefill_rows_gqa(q, k, v, variant, 5, 0.4)
    b = oracle_mod.prefill_rows(q, k, v, variant, 5, 0.4)
    assert np.array_equal(a, b)


def test_gqa_heads_of_a_group_see_the_same_keys(oracle_mod):
    # Two query heads of one group with equal queries give equal outputs; the same queries
    # in another group (other keys) give different ones.
    q, k, v = _inputs(11, 1, 4, 2, 17, 8)
    q[0, 1] = q[0, 0]
    q[0, 2] = q[0, 0]
    out = oracle_mod.prefill_rows_gqa(q, k, v, "full")
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 2])


def test_gqa_rejects_bad_groups(oracle_mod):
    q, k, v = _inputs(3, 1, 4, 3, 5, 4)
    with pytest.raises(ValueError):
        oracle_mod.prefill_rows_gqa(q, k, v, "full")
    with pytest.raises(ValueError):
        oracle_mod.prefill_rows_gqa(q, k[:, :, :4], v, "full")
