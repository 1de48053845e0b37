"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs, element by element, with max abs <= 2e-2 and rel-L2 <= 5e-3.

Variants as in Table 1 of "Placement Is Free, Composition Is Not" (full, sliding,
differential); the causal property is audited as in its sec. 8.
"""
import numpy as np
import pytest

from gpu_util import (assert_close, device_tensors, make, run_layer, sample_rows, to_f64)
from heterogeneous_attention_mixer_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from heterogeneous_attention_mixer_amd import mixer as M
    M.lib()
    return torch


def _oracle(oracle_mod, inp, variant, W, lam, rows=None):
    return oracle_mod.prefill_rows(inp.q, inp.k, inp.v, variant, W, lam, rows)


# ------------------------------------------------------------- small, every row compared

def test_fp32_small_full(torch_cuda, oracle_mod):
    """fp32 inputs, B=1, H=2, L=256, d=64, full causal (rounded to bf16 on load)."""
    w = synth.WORKLOADS["full_fp32_L256_d64"]
    inp = make(w["seed"], w["B"], w["H"], w["L"], w["d"], "f32")
    out = run_layer(device_tensors(inp), "full")
    assert out.dtype == torch_cuda.float32
    assert_close(to_f64(out), _oracle(oracle_mod, inp, "full", 0, 0.0), "fp32 L256 d64")


SMALL = []
for d in (64, 128):
    for L in (1, 2, 63, 64, 128, 129, 777):
        SMALL.append(("full", d, 2, 3, L, 0, 0.0))
        SMALL.append(("differential", d, 1, 3, L, 0, 0.8))
    for L, W in ((777, 1), (777, 37), (777, 64), (777, 100), (777, 128), (777, 777),
                 (777, 2000), (300, 129), (129, 63)):
        SMALL.append(("sliding", d, 1, 3, L, W, 0.0))
    SMALL.append(("differential", d, 2, 2, 300, 0, 0.0))
    SMALL.append(("differential", d, 1, 2, 300, 0, -0.3))


@pytest.mark.parametrize("variant,d,B,H,L,W,lam", SMALL)
def test_small_every_row(torch_cuda, oracle_mod, variant, d, B, H, L, W, lam):
    inp = make(1000 + L + d + W, B, H, L, d)
    out = run_layer(device_tensors(inp), variant, W, lam)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, variant, W, lam),
                 f"{variant} d={d} B={B} H={H} L={L} W={W} lam={lam}")


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 200, 0.0),
                                           ("differential", 0, 0.8)])
def test_fp32_every_variant(torch_cuda, oracle_mod, variant, W, lam):
    inp = make(77, 1, 2, 500, 128, "f32")
    out = run_layer(device_tensors(inp), variant, W, lam)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, variant, W, lam), variant)


# ------------------------------------------------- full workload sizes, sampled rows

FULLSIZE = [
    ("sliding_W1024_L8192", 256),
    ("full_L2048", 256),
    ("full_L8192", 256),
    ("differential_L8192", 256),
    ("full_L32768", 64),
    ("differential_L32768", 64),
]


@pytest.mark.parametrize("name,n_random", FULLSIZE)
def test_full_size_sampled_rows(torch_cuda, oracle_mod, name, n_random):
    w = synth.WORKLOADS[name]
    inp = make(w["seed"], w["B"], w["H"], w["L"], w["d"])
    out = run_layer(device_tensors(inp), w["variant"], w["window"], w["lam"])
    got = out.float()
    assert bool(torch_cuda.isfinite(got).all()), "non-finite output"
    rows = sample_rows(w["L"], seed=w["seed"], n_random=n_random)
    ref = _oracle(oracle_mod, inp, w["variant"], w["window"], w["lam"], rows)
    assert_close(to_f64(out[:, :, rows]), ref, name)


# ------------------------------------------- many heads: several heads per XCD block

# B*H a multiple of 8 gives each XCD a contiguous block of B*H/8 heads; the shapes above
# give it two. These give it 6, 8 and 9, with a ragged sequence length.
MANY_HEADS = [("full", 2, 24, 1000, 0, 0.0), ("sliding", 2, 32, 777, 200, 0.0),
              ("differential", 1, 72, 640, 0, 0.8)]


@pytest.mark.parametrize("variant,B,H,L,W,lam", MANY_HEADS)
def test_many_heads_sampled_rows(torch_cuda, oracle_mod, variant, B, H, L, W, lam):
    inp = make(900 + H, B, H, L, 128)
    out = run_layer(device_tensors(inp), variant, W, lam)
    rows = sample_rows(L, seed=H, n_random=24, edge=8)
    ref = _oracle(oracle_mod, inp, variant, W, lam, rows)
    assert_close(to_f64(out[:, :, rows]), ref, f"{variant} B={B} H={H} L={L}")


@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 30, 0.0),
                                           ("differential", 0, 0.5)])
def test_many_small_heads_every_row(torch_cuda, oracle_mod, variant, W, lam):
    """512 (batch, head) slices of 100 tokens, one query tile each: 512 workgroups over a
    head count that is a multiple of 8 (64 heads per XCD block)."""
    inp = make(950, 8, 64, 100, 64)
    out = run_layer(device_tensors(inp), variant, W, lam)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, variant, W, lam), f"{variant} 8x64 heads")


# --------------------------------------- key magnitudes that move the reference max

def _scale_keys(inp, factors):
    """Key j times factors[j], rounded to bf16 again: in place, on both the values the oracle
    sees and the bits the device receives."""
    bits = synth.round_to_bf16_bits((inp.k * factors[None, None, :, None]).astype(np.float32))
    inp.k[...] = synth.bf16_bits_to_f32(bits)
    inp.k_bits[...] = bits


# Rising: later keys score up to 7x higher, so a row's reference max keeps moving past the
# rescale threshold. Falling: the first keys dominate and later weights underflow. Spikes:
# every 97th key 12x larger.
KEY_PROFILES = {
    "rising": lambda L: 1.0 + 6.0 * np.arange(L) / L,
    "falling": lambda L: 7.0 - 6.0 * np.arange(L) / L,
    "spikes": lambda L: np.where(np.arange(L) % 97 == 50, 12.0, 1.0),
}


@pytest.mark.parametrize("profile", sorted(KEY_PROFILES))
@pytest.mark.parametrize("variant,d,W,lam", [("full", 128, 0, 0.0), ("sliding", 128, 300, 0.0),
                                             ("differential", 128, 0, 0.8),
                                             ("full", 64, 0, 0.0),
                                             ("differential", 64, 0, -0.5)])
def test_moving_reference_max_every_row(torch_cuda, oracle_mod, profile, variant, d, W, lam):
    L = 777
    inp = make(970 + d, 1, 2, L, d)
    _scale_keys(inp, KEY_PROFILES[profile](L))
    out = run_layer(device_tensors(inp), variant, W, lam)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, variant, W, lam),
                 f"{profile} keys, {variant} d={d}")


@pytest.mark.parametrize("profile", sorted(KEY_PROFILES))
@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 200, 0.0),
                                           ("differential", 0, 0.8)])
def test_moving_reference_max_fp32_entry(torch_cuda, oracle_mod, profile, variant, W, lam):
    """The same key profiles through the fp32 entry point (its own kernel, which rounds to
    bf16 as it stages; the oracle takes the fp32 values)."""
    L = 500
    inp = make(980, 1, 2, L, 128, "f32")
    inp.k[...] = (inp.k * KEY_PROFILES[profile](L)[None, None, :, None]).astype(np.float32)
    out = run_layer(device_tensors(inp), variant, W, lam)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, variant, W, lam),
                 f"fp32 {profile} keys, {variant}")


# ------------------------------------------------------------------------ invariants

@pytest.mark.parametrize("variant,W,lam,expect", [("full", 0, 0.0, 1.0),
                                                  ("sliding", 100, 0.0, 1.0),
                                                  ("differential", 0, 0.8, 0.2),
                                                  ("differential", 0, -0.3, 1.3)])
def test_unit_values_give_row_sums(torch_cuda, variant, W, lam, expect):
    inp = make(5, 1, 4, 1000, 128)
    q, k, v = device_tensors(inp)
    v = torch_cuda.ones_like(v)
    out = run_layer((q, k, v), variant, W, lam).float()
    # 4e-3 for the bf16-rounded probabilities, plus half a bf16 ulp for the output rounding
    assert float((out - expect).abs().max()) <= 4e-3 + abs(expect) * 2.0**-8


@pytest.mark.parametrize("L,W", [(777, 777), (777, 5000), (1000, 1000), (128, 128)])
def test_window_at_least_L_is_full_bitwise(torch_cuda, L, W):
    t = device_tensors(make(6, 1, 3, L, 128))
    a = run_layer(t, "sliding", W)
    b = run_layer(t, "full")
    assert torch_cuda.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_window_one_is_v_bitwise(torch_cuda, d):
    t = device_tensors(make(7, 2, 2, 333, d))
    assert torch_cuda.equal(run_layer(t, "sliding", 1), t[2])


def test_differential_equal_halves(torch_cuda, oracle_mod):
    """With q1 = q2 and k1 = k2: diff(lambda) = (1 - lambda) diff(0), and diff(0) is plain
    causal attention on the half-width scores with full-width values."""
    L, d = 600, 128
    inp = make(8, 1, 2, L, d)
    for x in (inp.q, inp.k):
        x[..., d // 2:] = x[..., :d // 2]
    for b in (inp.q_bits, inp.k_bits):
        b[..., d // 2:] = b[..., :d // 2]
    t = device_tensors(inp)
    d0 = to_f64(run_layer(t, "differential", 0, 0.0))
    d8 = to_f64(run_layer(t, "differential", 0, 0.8))
    assert_close(d8, 0.2 * d0, "diff(0.8) vs 0.2 diff(0)")
    for h in range(2):
        ref = oracle_mod.attention_general(inp.q[0, h, :, :d // 2], inp.k[0, h, :, :d // 2],
                                           inp.v[0, h], 1.0 / np.sqrt(d // 2))
        assert_close(d0[0, h], ref, f"diff(0) head {h}")


# ---------------------------------------------------- causal audit (sec. 8) on the GPU

@pytest.mark.parametrize("variant,W,lam", [("full", 0, 0.0), ("sliding", 70, 0.0),
                                           ("differential", 0, 0.8)])
@pytest.mark.parametrize("t", [0, 63, 64, 200, 511])
def test_future_inputs_do_not_change_past_rows(torch_cuda, variant, W, lam, t):
    L = 700
    inp = make(9, 1, 2, L, 128)
    a = run_layer(device_tensors(inp), variant, W, lam)
    rng = np.random.default_rng(10 + t)
    for bits in (inp.q_bits, inp.k_bits, inp.v_bits):
        bits[:, :, t + 1:] = rng.integers(0, 2**16, size=bits[:, :, t + 1:].shape,
                                          dtype=np.uint16) & 0x3FFF  # finite, |x| < 2
    b = run_layer(device_tensors(inp), variant, W, lam)
    assert torch_cuda.equal(a[:, :, :t + 1], b[:, :, :t + 1])
    assert not torch_cuda.equal(a[:, :, t + 1:], b[:, :, t + 1:])


def test_keys_outside_window_do_not_change_row(torch_cuda):
    L, W, i = 700, 90, 500
    inp = make(11, 1, 2, L, 128)
    a = run_layer(device_tensors(inp), "sliding", W)
    inp.k_bits[:, :, :i - W + 1] = 0x3F80  # 1.0
    inp.v_bits[:, :, :i - W + 1] = 0xC000  # -2.0
    b = run_layer(device_tensors(inp), "sliding", W)
    assert torch_cuda.equal(a[:, :, i:], b[:, :, i:])  # rows >= i see none of them


# ------------------------------------------- determinism, coverage of out, no stray writes

# The key loop's loads are inline assembly whose completion the kernel tracks itself (a
# vmcnt wait and a barrier before any tile is read). A schedule that broke that (a load in
# flight past its wait, a register reused under it) shows up first as results that change
# from run to run, so every shape the bench times, a ragged length, the key-split path
# (one workgroup per CU or fewer) and both head dims run three times and must agree bitwise.
REPRO = [(variant, W, lam, B, H, L, d)
         for variant, W, lam in (("full", 0, 0.0), ("sliding", 1024, 0.0),
                                 ("differential", 0, 0.8))
         for B, H, L, d in ((1, 16, 8192, 128), (1, 16, 4096, 128), (1, 5, 3001, 128),
                            (1, 16, 2048, 128), (2, 3, 1500, 64))]


@pytest.mark.parametrize("variant,W,lam,B,H,L,d", REPRO)
def test_bitwise_reproducible(torch_cuda, variant, W, lam, B, H, L, d):
    t = device_tensors(make(12, B, H, L, d))
    a = run_layer(t, variant, W, lam)
    for _ in range(2):
        assert torch_cuda.equal(a, run_layer(t, variant, W, lam))


# The full and sliding layers split each row block's keys over two waves when the grid holds
# at most one workgroup per CU (B*H*ceil(L/128) <= 256 on MI355X). Both sides of that
# boundary, against the oracle on sampled rows.
SPLIT_EDGE = [("full", 0, 2, 16384, 128), ("full", 0, 2, 16385, 128),
              ("sliding", 700, 2, 16384, 128), ("sliding", 700, 2, 16385, 128),
              ("full", 0, 4, 8192, 64), ("full", 0, 4, 8193, 64)]


@pytest.mark.parametrize("variant,W,H,L,d", SPLIT_EDGE)
def test_key_split_boundary_sampled_rows(torch_cuda, oracle_mod, variant, W, H, L, d):
    inp = make(31 + L % 7, 1, H, L, d)
    out = run_layer(device_tensors(inp), variant, W, 0.0)
    rows = sample_rows(L, seed=L, n_random=96, edge=40)
    ref = _oracle(oracle_mod, inp, variant, W, 0.0, rows)
    assert_close(to_f64(out[:, :, rows]), ref, f"{variant} H={H} L={L} d={d}")


# Full causal runs the phase-separated kernel (256-row workgroups) when its grid holds more
# than one of them per CU (B*H*ceil(L/256) > 256 on MI355X), else the pipelined kernel. Both
# sides of that boundary at both head dims, against the oracle on sampled rows.
PHASE_EDGE = [(2, 32768, 128), (2, 32769, 128), (4, 16384, 64), (4, 16385, 64)]


@pytest.mark.parametrize("H,L,d", PHASE_EDGE)
def test_full_phase_kernel_boundary_sampled_rows(torch_cuda, oracle_mod, H, L, d):
    inp = make(41 + L % 7, 1, H, L, d)
    out = run_layer(device_tensors(inp), "full", 0, 0.0)
    rows = sample_rows(L, seed=L, n_random=64, edge=40)
    ref = _oracle(oracle_mod, inp, "full", 0, 0.0, rows)
    assert_close(to_f64(out[:, :, rows]), ref, f"full H={H} L={L} d={d}")


# The phase-separated full kernel on ragged lengths (not a multiple of its 256 rows or of
# the 64-key tile), every row against the oracle.
@pytest.mark.parametrize("B,H,L,d", [(2, 80, 333, 128), (4, 33, 700, 64)])
def test_full_phase_kernel_every_row(torch_cuda, oracle_mod, B, H, L, d):
    inp = make(43, B, H, L, d)
    out = run_layer(device_tensors(inp), "full", 0, 0.0)
    assert_close(to_f64(out), _oracle(oracle_mod, inp, "full", 0, 0.0),
                 f"full B={B} H={H} L={L} d={d}")


@pytest.mark.parametrize("L", [1, 255, 257, 1000])
def test_full_phase_kernel_writes_every_row_and_nothing_else(torch_cuda, L):
    import torch
    B, H, d = 2, 130, 128  # B*H*ceil(L/256) > 256: the phase-separated kernel
    inp = make(14, B, H, L, d)
    q, k, v = device_tensors(inp)
    n = B * H * L * d
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[n:] = 1024.0
    out = buf[:n].view(B, H, L, d)
    run_layer((q, k, v), "full", 0, 0.0, out=out)
    assert bool(torch.isfinite(out.float()).all())
    assert bool((buf[n:].float() == 1024.0).all())


@pytest.mark.parametrize("L", [1, 127, 129, 1000])
@pytest.mark.parametrize("variant", ["full", "sliding", "differential"])
def test_every_row_written_and_nothing_else(torch_cuda, variant, L):
    import torch
    B, H, d = 2, 3, 128
    inp = make(13, B, H, L, d)
    q, k, v = device_tensors(inp)
    n = B * H * L * d
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[n:] = 1024.0
    out = buf[:n].view(B, H, L, d)
    run_layer((q, k, v), variant, 50, 0.5, out=out)
    assert bool(torch.isfinite(out.float()).all())
    assert bool((buf[n:].float() == 1024.0).all())
