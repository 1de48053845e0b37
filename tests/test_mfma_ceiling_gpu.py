"""The matrix-core ceiling measurement (a measurement aid, not part of the method): its chains
hold exactly the documented products, element by element against numpy in fp64, which also
pins the v_mfma_f32_32x32x16_bf16 operand and result lane layout the prefill kernel relies on
(A: lane l holds row l % 32, k = 8*(l/32) + [0, 8); B: column l % 32, the same k; result
element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32)."""
import numpy as np
import pytest

from heterogeneous_attention_mixer_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from heterogeneous_attention_mixer_amd import mixer as M
    M.lib()
    return torch


def _matrices(frag_set):
    """(4 A matrices 32 x 16, 4 B matrices 16 x 32) in fp64 from one set (8, 64, 8) of bits."""
    x = synth.bf16_bits_to_f32(frag_set).astype(np.float64)
    lanes = np.arange(64)
    A, B = [], []
    for f in range(4):
        a = np.zeros((32, 16))
        b = np.zeros((16, 32))
        for l in lanes:
            a[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = x[f, l]
            b[8 * (l // 32):8 * (l // 32) + 8, l % 32] = x[4 + f, l]
        A.append(a)
        B.append(b)
    return A, B


def _expected_sink(frags, blocks, iters):
    nsets = frags.shape[0]
    r = np.arange(16)[:, None]
    l = np.arange(64)[None, :]
    rows = 8 * (r // 4) + 4 * (l // 32) + r % 4          # (16, 64)
    cols = np.broadcast_to(l % 32, rows.shape)
    out = np.zeros((blocks * 4, 4, 16, 64))
    mats = [_matrices(frags[s]) for s in range(nsets)]
    for w in range(blocks * 4):
        A, B = mats[w % nsets]
        for c in range(4):
            D = sum(A[(u + c) % 4] @ B[(u + 2 * c) % 4] for u in range(4)) * (iters // 4)
            out[w, c] = D[rows, cols]
    return out


@pytest.mark.parametrize("blocks,iters,nsets", [(3, 4, 1), (8, 16, 5), (2, 64, 8)])
def test_chains_hold_the_documented_products(torch_cuda, blocks, iters, nsets):
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    bits = synth.make_mfma_fragments(700 + nsets, nsets)
    frags = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    n = blocks * M.CEILING_SINK_PER_BLOCK
    sink = torch.full((n + 64,), float("nan"), dtype=torch.float32, device="cuda")
    M.mixer_mfma_ceiling_async(frags, sink, blocks, iters)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    assert np.isnan(got[n:]).all(), "wrote past the documented sink size"
    want = _expected_sink(bits, blocks, iters).reshape(-1)
    # bf16 x bf16 products are exact in fp32; the error is fp32 accumulation only.
    np.testing.assert_allclose(got[:n], want, rtol=1e-5, atol=1e-4 * iters)


def test_two_calls_are_bitwise_equal(torch_cuda):
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    bits = synth.make_mfma_fragments(3, 4)
    frags = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    a = torch.empty(16 * M.CEILING_SINK_PER_BLOCK, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    M.mixer_mfma_ceiling_async(frags, a, 16, 40)
    M.mixer_mfma_ceiling_async(frags, b, 16, 40)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
