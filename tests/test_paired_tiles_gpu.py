"""GPU: full causal attention with paired query tiles.

When the grid holds at most one workgroup per CU and the sequence has an even number of
64-row query tiles, each workgroup takes a light tile and its mirror (tiles t and n-1-t of
n), with the keys of every 32-row block split over two waves, and the light tile's waves stop
their matrix work once past their last visible key. Every row against the fp64 oracle, on
ragged lengths, both head dims, grouped key/value heads, and the odd tile count that falls
back to unpaired workgroups. Causal attention as in Table 1 of "Placement Is Free,
Composition Is Not" (full row).
"""
import pytest

from gpu_util import assert_close, device_tensors, make, run_layer, to_f64
from heterogeneous_attention_mixer_amd import mixer as M
from heterogeneous_attention_mixer_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.lib()
    return torch


def _tiles64(L):
    return (L + 63) // 64


# (B, H, L, d): B*H*ceil(L/128) <= 256 in every case. Even 64-row tile counts (paired), some
# with a partial last tile, and one odd count (unpaired key split).
CASES = [(1, 3, 128, 128), (2, 3, 1000, 128), (1, 5, 2000, 64), (1, 1, 1989, 128),
         (3, 2, 256, 64), (1, 16, 640, 128), (2, 2, 1088, 128), (1, 4, 1050, 128)]


@pytest.mark.parametrize("B,H,L,d", CASES)
def test_paired_tiles_every_row(torch_cuda, oracle_mod, B, H, L, d):
    assert B * H * ((L + 127) // 128) <= 256
    inp = make(500 + L + d, B, H, L, d)
    out = run_layer(device_tensors(inp), "full", 0, 0.0)
    ref = oracle_mod.prefill_rows(inp.q, inp.k, inp.v, "full", 0, 0.0)
    paired = _tiles64(L) % 2 == 0
    assert_close(to_f64(out), ref, f"full B={B} H={H} L={L} d={d} paired={paired}")


def test_case_list_covers_both_layouts():
    counts = [_tiles64(L) % 2 for _, _, L, _ in CASES]
    assert 0 in counts and 1 in counts
    assert any(L % 64 for _, _, L, _ in CASES if _tiles64(L) % 2 == 0)  # a ragged paired case


@pytest.mark.parametrize("d", [64, 128])
def test_paired_tiles_grouped_heads_every_row(torch_cuda, oracle_mod, d):
    import torch
    import numpy as np
    inp = synth.make_qkv_gqa(610 + d, 1, 8, 2, 1000, d)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(b)).view(torch.bfloat16).to("cuda")
               for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    out = torch.full_like(q, float("nan"))
    M.mixer_prefill_gqa_async(q, k, v, out, "full", 0, 0.0)
    torch.cuda.synchronize()
    ref = oracle_mod.prefill_rows_gqa(inp.q, inp.k, inp.v, "full", 0, 0.0)
    assert_close(to_f64(out), ref, f"gqa full d={d}")


@pytest.mark.parametrize("B,H,L,d", [(2, 3, 1000, 128), (1, 5, 2000, 64)])
def test_paired_tiles_bitwise_reproducible(torch_cuda, B, H, L, d):
    t = device_tensors(make(12, B, H, L, d))
    a = run_layer(t, "full", 0, 0.0)
    for _ in range(2):
        assert torch_cuda.equal(a, run_layer(t, "full", 0, 0.0))
