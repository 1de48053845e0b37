"""GPU parity of the grouped key/value-head entry point (``mixer_prefill_gqa_async``) against
the fp64 oracle (``prefill_rows_gqa``).

Grouped heads are the model's attention shape in "Placement Is Free, Composition Is Not"
(Table 2, sec. 4.1: 16 heads over 4 KV heads, head_dim 128). Small cases compare every row;
the model shape at L=8192 compares sampled rows of every head.
"""
import numpy as np
import pytest

from gpu_util import assert_close, run_layer, sample_rows, to_f64
from heterogeneous_attention_mixer_amd import mixer as M
from heterogeneous_attention_mixer_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()
    return torch


def _dev(inp):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(b)).view(torch.bfloat16).to("cuda")
            for b in (inp.q_bits, inp.k_bits, inp.v_bits)]


def _run_gqa(t, variant, W, lam):
    import torch
    q, k, v = t
    out = torch.full_like(q, float("nan"))
    M.mixer_prefill_gqa_async(q, k, v, out, variant, W, lam)
    torch.cuda.synchronize()
    return out


SMALL = []
for d in (64, 128):
    for B, H, Hkv, L in ((1, 4, 2, 129), (2, 4, 1, 63), (1, 8, 2, 300)):
        SMALL.append(("full", d, B, H, Hkv, L, 0, 0.0))
        SMALL.append(("sliding", d, B, H, Hkv, L, 37, 0.0))
        SMALL.append(("differential", d, B, H, Hkv, L, 0, 0.8))
# B*H = 64: each XCD takes a block of 8 query heads, i.e. two whole groups of 4.
for variant, W, lam in (("full", 0, 0.0), ("sliding", 50, 0.0), ("differential", 0, 0.8)):
    SMALL.append((variant, 128, 2, 32, 8, 200, W, lam))


@pytest.mark.parametrize("variant,d,B,H,Hkv,L,W,lam", SMALL)
def test_gqa_small_every_row(torch_cuda, oracle_mod, variant, d, B, H, Hkv, L, W, lam):
    inp = synth.make_qkv_gqa(2000 + L + d + H + Hkv, B, H, Hkv, L, d)
    out = _run_gqa(_dev(inp), variant, W, lam)
    ref = oracle_mod.prefill_rows_gqa(inp.q, inp.k, inp.v, variant, W, lam)
    assert_close(to_f64(out), ref, f"gqa {variant} d={d} B={B} H={H} Hkv={Hkv} L={L}")


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 100, 0.0),
                                           ("differential", 0, -0.4)])
def test_gqa_with_one_head_per_group_is_bitwise_the_plain_call(torch_cuda, variant, W, lam):
    import torch
    inp = synth.make_qkv(77, 2, 3, 200, 128)
    t = _dev(inp)
    a = _run_gqa(t, variant, W, lam)
    b = run_layer(t, variant, W, lam)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_gqa_heads_of_a_group_share_keys(torch_cuda):
    # Equal queries in two heads of one group give bitwise equal outputs.
    import torch
    inp = synth.make_qkv_gqa(91, 1, 8, 2, 333, 128)
    t = _dev(inp)
    t[0][0, 1] = t[0][0, 0]
    t[0][0, 5] = t[0][0, 0]
    out = _run_gqa(t, "full", 0, 0.0)
    assert torch.equal(out[0, 0], out[0, 1])        # heads 0, 1: group 0
    assert not torch.equal(out[0, 0], out[0, 5])    # head 5: group 1, other keys


@pytest.mark.parametrize("variant", ["full", "sliding", "differential"])
def test_gqa_model_shape_sampled_rows(torch_cuda, oracle_mod, variant):
    g = synth.GQA
    W = g["window"] if variant == "sliding" else 0
    lam = g["lam"] if variant == "differential" else 0.0
    inp = synth.make_qkv_gqa(g["seed0"] + M.VARIANTS[variant], g["B"], g["H"], g["Hkv"],
                             g["L"], g["d"])
    out = to_f64(_run_gqa(_dev(inp), variant, W, lam))
    rows = sample_rows(g["L"], 31, n_random=96, edge=32)
    ref = oracle_mod.prefill_rows_gqa(inp.q, inp.k, inp.v, variant, W, lam, rows)
    assert_close(out[:, :, rows, :], ref, f"gqa model shape {variant}")
