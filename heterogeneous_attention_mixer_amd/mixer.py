"""Thin ctypes binding of libmixer.so (the C ABI declared in include/mixer.h).

Argument marshalling only: every step of the layer runs in the HIP kernels. PyTorch supplies
device memory (``Tensor.data_ptr()``) and the stream (the current torch stream of the
tensors' device). The functions keep the C names; shapes are read from the tensors.

The library is loaded on first use. If it has not been built this raises ``MixerError``;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmixer.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mixer.h")

FULL, SLIDING, DIFFERENTIAL = 0, 1, 2
VARIANTS = {"full": FULL, "sliding": SLIDING, "differential": DIFFERENTIAL}

OK, EINVAL, EUNSUPPORTED, ENOTLATIN, EHIP = 0, -1, -2, -3, -4


class MixerError(RuntimeError):
    """A negative mixer_status, or a library that cannot be loaded."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmixer.so with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MixerError(f"{LIB_PATH} is not built; run "
                         "`python -m heterogeneous_attention_mixer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    ip = ctypes.POINTER(ctypes.c_int)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    L.mixer_prefill_async.argtypes = [vp, vp, vp, vp, ci, ci, cf, ci, ci, ci, ci, vp]
    L.mixer_prefill_gqa_async.argtypes = [vp, vp, vp, vp, ci, ci, cf, ci, ci, ci, ci, ci, vp]
    L.mixer_prefill.argtypes = [vp, vp, vp, vp, ci, ci, cf, ci, ci, ci, ci]
    L.mixer_prefill_f32_async.argtypes = [vp, vp, vp, vp, ci, ci, cf, ci, ci, ci, ci, vp]
    L.mixer_latin_build.argtypes = [ci, ip, ip]
    L.mixer_latin_check.argtypes = [ci, ip]
    L.mixer_stack_prefill.argtypes = [ci, ip, vpp, vpp, vpp, vpp, ci, cf, ci, ci, ci, ci, vp,
                                      vpp]
    L.mixer_layers_prefill.argtypes = [ci, ip, vpp, vpp, vpp, vpp, ci, cf, ci, ci, ci, ci, vp,
                                       vpp]
    L.mixer_mfma_ceiling_async.argtypes = [vp, ci, vp, ci, ci, vp]
    L.mixer_strerror.argtypes = [ci]
    L.mixer_strerror.restype = ctypes.c_char_p
    for name in ("mixer_prefill_async", "mixer_prefill_gqa_async", "mixer_prefill",
                 "mixer_prefill_f32_async",
                 "mixer_latin_build", "mixer_latin_check", "mixer_stack_prefill",
                 "mixer_layers_prefill", "mixer_mfma_ceiling_async"):
        getattr(L, name).restype = ci
    _lib = L
    return L


def header_symbols() -> list:
    """Every function name include/mixer.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mixer_\w+)\s*\(", text)))


def mixer_strerror(status: int) -> str:
    return lib().mixer_strerror(int(status)).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise MixerError(f"{what}: {mixer_strerror(rc)} (status {rc})", rc)


def _variant(v) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


def _stream_of(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(q, k, v, out, dtype):
    import torch
    ts = (q, k, v, out)
    if any(not isinstance(t, torch.Tensor) for t in ts):
        raise TypeError("q, k, v, out must be torch tensors")
    if any(t.device.type != "cuda" for t in ts) or len({t.device for t in ts}) != 1:
        raise MixerError("q, k, v, out must live on one GPU", EINVAL)
    if any(t.dtype != dtype for t in ts):
        raise MixerError(f"q, k, v, out must be {dtype}", EINVAL)
    if any(t.dim() != 4 or t.shape != q.shape for t in ts):
        raise MixerError("q, k, v, out must share one [B, H, L, d] shape", EINVAL)
    if any(not t.is_contiguous() for t in ts):
        raise MixerError("q, k, v, out must be contiguous", EINVAL)
    return tuple(int(x) for x in q.shape)


def mixer_prefill_async(q, k, v, out, variant, window: int = 0, lam: float = 0.0,
                        stream=None):
    """One bf16 layer on tensors [B, H, L, d]; enqueued on ``stream`` (a torch stream, or
    the current stream of the tensors' device). Returns ``out``."""
    import torch
    B, H, L, d = _shape(q, k, v, out, torch.bfloat16)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(q)
    with torch.cuda.device(q.device):
        rc = lib().mixer_prefill_async(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       out.data_ptr(), _variant(variant), int(window),
                                       float(lam), B, H, L, d, s)
    _check(rc, "mixer_prefill_async")
    return out


def mixer_prefill_gqa_async(q, k, v, out, variant, window: int = 0, lam: float = 0.0,
                            stream=None):
    """One bf16 layer with grouped key/value heads: q and out [B, H, L, d], k and v
    [B, Hkv, L, d] with Hkv dividing H. Returns ``out``."""
    import torch
    ts = (q, k, v, out)
    if any(not isinstance(t, torch.Tensor) for t in ts):
        raise TypeError("q, k, v, out must be torch tensors")
    if any(t.device.type != "cuda" for t in ts) or len({t.device for t in ts}) != 1:
        raise MixerError("q, k, v, out must live on one GPU", EINVAL)
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise MixerError("q, k, v, out must be torch.bfloat16", EINVAL)
    if any(t.dim() != 4 for t in ts) or out.shape != q.shape or k.shape != v.shape:
        raise MixerError("q, out must share [B, H, L, d]; k, v [B, Hkv, L, d]", EINVAL)
    B, H, L, d = (int(x) for x in q.shape)
    if k.shape[0] != B or k.shape[2] != L or k.shape[3] != d:
        raise MixerError("k, v must be [B, Hkv, L, d] with q's B, L and d", EINVAL)
    if any(not t.is_contiguous() for t in ts):
        raise MixerError("q, k, v, out must be contiguous", EINVAL)
    Hkv = int(k.shape[1])
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(q)
    with torch.cuda.device(q.device):
        rc = lib().mixer_prefill_gqa_async(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), _variant(variant), int(window),
                                           float(lam), B, H, Hkv, L, d, s)
    _check(rc, "mixer_prefill_gqa_async")
    return out


def mixer_prefill(q, k, v, out, variant, window: int = 0, lam: float = 0.0):
    """One bf16 layer on the legacy default stream (the C entry point of the same name)."""
    import torch
    B, H, L, d = _shape(q, k, v, out, torch.bfloat16)
    with torch.cuda.device(q.device):
        rc = lib().mixer_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 _variant(variant), int(window), float(lam), B, H, L, d)
    _check(rc, "mixer_prefill")
    return out


def mixer_prefill_f32_async(q, k, v, out, variant, window: int = 0, lam: float = 0.0,
                            stream=None):
    """One layer on fp32 tensors: scores from split (high + low bf16) q and k, v rounded to
    bf16 on load, fp32 result."""
    import torch
    B, H, L, d = _shape(q, k, v, out, torch.float32)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(q)
    with torch.cuda.device(q.device):
        rc = lib().mixer_prefill_f32_async(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), _variant(variant), int(window),
                                           float(lam), B, H, L, d, s)
    _check(rc, "mixer_prefill_f32_async")
    return out


def prefill(q, k, v, variant="full", window: int = 0, lam: float = 0.0, out=None):
    """Convenience: allocates ``out`` and dispatches on dtype (bf16 or fp32)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if q.dtype == torch.float32:
        return mixer_prefill_f32_async(q, k, v, out, variant, window, lam)
    return mixer_prefill_async(q, k, v, out, variant, window, lam)


def mixer_latin_build(base) -> list:
    """The cyclic Latin square of ``base`` (N entries), flat row-major (N*N entries)."""
    n = len(base)
    b = (ctypes.c_int * max(n, 1))(*[int(x) for x in base])
    s = (ctypes.c_int * max(n * n, 1))()
    _check(lib().mixer_latin_build(n, b, s), "mixer_latin_build")
    return list(s)[: n * n]


def mixer_latin_check(n: int, sched) -> bool:
    """True iff the flat row-major n x n schedule is a Latin square."""
    s = (ctypes.c_int * max(len(sched), 1))(*[int(x) for x in sched])
    rc = lib().mixer_latin_check(int(n), s)
    if rc < 0:
        _check(rc, "mixer_latin_check")
    return rc == 1


def _layer_args(m, variants, qs, ks, vs, outs, events):
    import torch
    if m < 1:
        raise MixerError("at least one layer is required", EINVAL)
    if not (len(variants) == len(qs) == len(ks) == len(vs) == len(outs) == m):
        raise MixerError("variant and tensor lists must hold one entry per layer", EINVAL)
    B, H, L, d = _shape(qs[0], ks[0], vs[0], outs[0], torch.bfloat16)
    for t in zip(qs, ks, vs, outs):
        _shape(*t, torch.bfloat16)
        if t[0].shape != qs[0].shape or t[0].device != qs[0].device:
            raise MixerError("every layer must share one shape and device", EINVAL)
    arr = lambda ts: (ctypes.c_void_p * m)(*[t.data_ptr() for t in ts])  # noqa: E731
    s = (ctypes.c_int * m)(*[_variant(x) for x in variants])
    ev = None
    if events is not None:
        if len(events) != m + 1:
            raise MixerError("events must hold one entry per layer plus one", EINVAL)
        ev = (ctypes.c_void_p * (m + 1))(*[None if e is None else
                                           e if isinstance(e, int) else e.cuda_event
                                           for e in events])
    return (B, H, L, d), s, arr(qs), arr(ks), arr(vs), arr(outs), ev


def mixer_stack_prefill(n: int, sched, qs, ks, vs, outs, window: int = 0, lam: float = 0.0,
                        events=None, stream=None):
    """Runs the n*n layers of a Latin schedule back to back on one stream. ``qs`` .. ``outs``
    are sequences of n*n bf16 tensors of one shape; ``events`` optionally n*n + 1 entries,
    each an event that the library records at that point (before layer 0, after each layer):
    a created ``torch.cuda.Event``, an object with a ``cuda_event`` handle, or a raw
    hipEvent_t as an int; or None to record nothing there."""
    import torch
    (B, H, L, d), s, q, k, v, o, ev = _layer_args(n * n, sched, qs, ks, vs, outs, events)
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(qs[0])
    with torch.cuda.device(qs[0].device):
        rc = lib().mixer_stack_prefill(n, s, q, k, v, o, int(window), float(lam), B, H, L, d,
                                       st, ev)
    _check(rc, "mixer_stack_prefill")
    return outs


def mixer_layers_prefill(variants, qs, ks, vs, outs, window: int = 0, lam: float = 0.0,
                         events=None, stream=None):
    """Runs len(variants) layers of any variants back to back on one stream (no Latin check);
    arguments as for ``mixer_stack_prefill``."""
    import torch
    m = len(variants)
    (B, H, L, d), s, q, k, v, o, ev = _layer_args(m, variants, qs, ks, vs, outs, events)
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(qs[0])
    with torch.cuda.device(qs[0].device):
        rc = lib().mixer_layers_prefill(m, s, q, k, v, o, int(window), float(lam), B, H, L, d,
                                        st, ev)
    _check(rc, "mixer_layers_prefill")
    return outs


CEILING_SET_ELEMS = 8 * 64 * 8      # bf16 elements per fragment set
CEILING_SINK_PER_BLOCK = 4 * 4 * 16 * 64  # floats written per workgroup


def mixer_mfma_ceiling_async(frags, sink, blocks: int, iters: int, stream=None):
    """Measurement aid (not part of the method): the matrix-core ceiling kernel.
    ``frags`` is a contiguous bf16 device tensor holding whole fragment sets (8 x 64 x 8
    elements each), ``sink`` a contiguous fp32 device tensor of at least
    blocks * 4 * 4 * 16 * 64 elements. One call executes blocks * 16 * iters MFMAs of
    32768 flops. Returns ``sink``."""
    import torch
    if not (isinstance(frags, torch.Tensor) and isinstance(sink, torch.Tensor)):
        raise TypeError("frags and sink must be torch tensors")
    if frags.dtype != torch.bfloat16 or sink.dtype != torch.float32:
        raise MixerError("frags must be bf16 and sink fp32", EINVAL)
    if frags.device.type != "cuda" or sink.device != frags.device:
        raise MixerError("frags and sink must live on one GPU", EINVAL)
    if not (frags.is_contiguous() and sink.is_contiguous()):
        raise MixerError("frags and sink must be contiguous", EINVAL)
    if frags.numel() == 0 or frags.numel() % CEILING_SET_ELEMS:
        raise MixerError("frags must hold whole fragment sets", EINVAL)
    if sink.numel() < int(blocks) * CEILING_SINK_PER_BLOCK:
        raise MixerError("sink is too small for that many workgroups", EINVAL)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream_of(frags)
    with torch.cuda.device(frags.device):
        rc = lib().mixer_mfma_ceiling_async(frags.data_ptr(), frags.numel() // CEILING_SET_ELEMS,
                                            sink.data_ptr(), int(blocks), int(iters), s)
    _check(rc, "mixer_mfma_ceiling_async")
    return sink
