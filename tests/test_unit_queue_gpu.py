"""GPU: the phase-separated kernel's persistent launch (one workgroup per CU taking
(head, query tile) units from per-XCD queues, stealing from the other queues at the end).

Every unit must be computed exactly where it belongs, the queue counters must be clean for
the next launch on the same stream, launches on different streams must not share counters,
and a stream that finds every queue slot taken must still get the right result (from the
one-workgroup-per-unit launch). Variants as in Table 1 of "Placement Is Free, Composition
Is Not" (full and differential run this kernel)."""
import numpy as np
import pytest

from gpu_util import assert_close, device_tensors, make, run_layer, to_f64

pytestmark = pytest.mark.gpu

# (variant, B, H, L, d, rows per unit): full takes 256-row units, the differential 128-row.
# B*H a multiple of 8 gives one queue per XCD, otherwise one queue; all have more units than
# the chip's 256 CUs, so they run persistent.
CASES = [
    ("full", 1, 16, 8192, 128, 256),
    ("full", 1, 3, 24577, 128, 256),
    ("full", 2, 4, 16384, 64, 256),
    ("differential", 1, 16, 4096, 128, 128),
    ("differential", 1, 5, 8192, 128, 128),
]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from heterogeneous_attention_mixer_amd import mixer as M
    M.lib()
    return torch


def _units(B, H, L, rows):
    return B * H * ((L + rows - 1) // rows)


def _lam(variant):
    return 0.8 if variant == "differential" else 0.0


@pytest.mark.parametrize("variant,B,H,L,d,rows", CASES)
def test_one_row_of_every_unit(torch_cuda, oracle_mod, variant, B, H, L, d, rows):
    cus = torch_cuda.cuda.get_device_properties(0).multi_processor_count
    assert _units(B, H, L, rows) > cus, "the case must run persistent"
    inp = make(71 + L % 11, B, H, L, d)
    out = run_layer(device_tensors(inp), variant, 0, _lam(variant))
    rng = np.random.default_rng(L + H)
    nq = (L + rows - 1) // rows
    # one seeded row inside every query tile, plus each tile's first and last row
    picks = set()
    for t in range(nq):
        lo, hi = t * rows, min(L, (t + 1) * rows) - 1
        picks |= {lo, hi, int(rng.integers(lo, hi + 1))}
    picked = np.array(sorted(picks), dtype=np.int64)
    ref = oracle_mod.prefill_rows(inp.q, inp.k, inp.v, variant, 0, _lam(variant), picked)
    assert_close(to_f64(out[:, :, picked]), ref, f"{variant} B={B} H={H} L={L} d={d}")
    assert bool(torch_cuda.isfinite(out.float()).all())


@pytest.mark.parametrize("variant", ["full", "differential"])
def test_repeated_launches_and_two_streams_agree_bitwise(torch_cuda, variant):
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    B, H, L, d = 1, 16, 8192, 128
    q, k, v = device_tensors(make(5, B, H, L, d))
    ref = run_layer((q, k, v), variant, 0, _lam(variant))
    outs = [torch.full_like(q, float("nan")) for _ in range(8)]
    # four back to back on the current stream (each must find its slot's counters at zero)
    for o in outs[:4]:
        M.mixer_prefill_async(q, k, v, o, variant, 0, _lam(variant))
    # four alternating over two more streams, with no wait between them
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    for i, o in enumerate(outs[4:]):
        M.mixer_prefill_async(q, k, v, o, variant, 0, _lam(variant), stream=s1 if i % 2 else s2)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"launch {i}"


@pytest.mark.parametrize("variant", ["full", "differential"])
def test_graph_replays_agree_bitwise(torch_cuda, variant):
    # A captured persistent launch keeps its capture stream's queue slot; every replay must
    # find the counters back at zero. Replays alternate with eager launches (on the current
    # stream's own slot) and synchronisations, and each is checked against the eager result.
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    B, H, L, d = 1, 16, 8192, 128
    q, k, v = device_tensors(make(8, B, H, L, d))
    ref = run_layer((q, k, v), variant, 0, _lam(variant))
    out = torch.full_like(q, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mixer_prefill_async(q, k, v, out, variant, 0, _lam(variant))
    other = torch.full_like(q, float("nan"))
    for i in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        other.fill_(float("nan"))
        M.mixer_prefill_async(q, k, v, other, variant, 0, _lam(variant))
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16)), f"eager {i}"


def test_per_thread_default_streams_of_two_threads_agree_bitwise(torch_cuda):
    # The per-thread default stream is one handle for a different stream in each host
    # thread; two threads launching on it at once must not share queue counters.
    import ctypes
    import threading
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    B, H, L, d = 1, 16, 8192, 128
    q, k, v = device_tensors(make(9, B, H, L, d))
    ref = run_layer((q, k, v), "full", 0, 0.0)
    outs = [[torch.full_like(q, float("nan")) for _ in range(4)] for _ in range(2)]
    torch.cuda.synchronize()
    per_thread = ctypes.c_void_p(2)  # hipStreamPerThread
    errs = []

    def launch(mine):
        try:
            torch.cuda.set_device(0)
            for o in mine:
                rc = M.lib().mixer_prefill_async(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 o.data_ptr(), 0, 0, 0.0, B, H, L, d,
                                                 per_thread)
                if rc != 0:
                    errs.append(rc)
        except Exception as e:  # reported below
            errs.append(e)

    threads = [threading.Thread(target=launch, args=(outs[i],)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i, mine in enumerate(outs):
        for j, o in enumerate(mine):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"thread {i} {j}"


def test_streams_beyond_the_queue_slots_fall_back(torch_cuda):
    # More streams than queue slots (256 per device): the later streams get the
    # one-workgroup-per-unit launch, which must give the same bits. The streams are made
    # through the HIP runtime (torch hands out a pool of 32). This takes every free slot of
    # the process, so it is the file's last test.
    import ctypes
    torch = torch_cuda
    from heterogeneous_attention_mixer_amd import mixer as M
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    B, H, L, d = 1, 16, 4608, 128  # 18 query tiles of 256 rows per head: 288 units
    q, k, v = device_tensors(make(6, B, H, L, d))
    ref = run_layer((q, k, v), "full", 0, 0.0)
    handles = []
    try:
        for _ in range(260):
            h = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(h)) == 0
            handles.append(h)
        outs = [torch.full_like(q, float("nan")) for _ in handles]
        torch.cuda.synchronize()  # inputs and the NaN fills are in place before any launch
        for h, o in zip(handles, outs):
            M.mixer_prefill_async(q, k, v, o, "full", 0, 0.0,
                                  stream=torch.cuda.ExternalStream(h.value))
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"stream {i}"
    finally:
        torch.cuda.synchronize()
        for h in handles:
            hip.hipStreamDestroy(h)
