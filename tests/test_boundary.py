"""The C-ABI library on a host without a GPU: it loads, exports every symbol mixer.h
declares, rejects every invalid argument with its code before touching the device, and its
pure-host Latin-square scheduler agrees exactly with the oracle's definition.

Source for the scheduler: "Placement Is Free, Composition Is Not", sec. 1, sec. 3.2 and
Table 7.
"""
import ctypes
import itertools
import math
import os

import pytest

from heterogeneous_attention_mixer_amd import build as mbuild
from heterogeneous_attention_mixer_amd import mixer as M
from oracle import latin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table7_schedules.txt")


@pytest.fixture(scope="module")
def lib():
    if mbuild.needs_build():
        mbuild.build()
    return M.lib()


def test_exports_every_declared_symbol(lib):
    names = M.header_symbols()
    assert set(names) >= {"mixer_prefill", "mixer_prefill_async", "mixer_prefill_f32_async",
                          "mixer_latin_build", "mixer_latin_check", "mixer_stack_prefill",
                          "mixer_strerror"}
    for n in names:
        assert hasattr(lib, n), n


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, 7, -99):
        s = M.mixer_strerror(code)
        assert isinstance(s, str) and s
    assert M.mixer_strerror(-3) != M.mixer_strerror(-1)


# Fake, never-dereferenced device addresses: every call below must fail validation first.
P = [0x10000000, 0x20000000, 0x30000000, 0x40000000]
OK_ARGS = dict(variant=0, window=0, lam=0.0, B=1, H=2, L=64, d=128)


def _call(lib, q=P[0], k=P[1], v=P[2], o=P[3], f32=False, stream=None, **kw):
    a = dict(OK_ARGS)
    a.update(kw)
    fn = lib.mixer_prefill_f32_async if f32 else lib.mixer_prefill_async
    return fn(q, k, v, o, a["variant"], a["window"], ctypes.c_float(a["lam"]), a["B"], a["H"],
              a["L"], a["d"], stream)


BAD = [
    (dict(q=None), M.EINVAL), (dict(k=None), M.EINVAL), (dict(v=None), M.EINVAL),
    (dict(o=None), M.EINVAL),
    (dict(B=0), M.EINVAL), (dict(H=0), M.EINVAL), (dict(L=0), M.EINVAL), (dict(L=-5), M.EINVAL),
    (dict(d=0), M.EINVAL),
    (dict(variant=3), M.EINVAL), (dict(variant=-1), M.EINVAL),
    (dict(variant=1, window=0), M.EINVAL), (dict(variant=1, window=-3), M.EINVAL),
    (dict(variant=2, lam=math.nan), M.EINVAL), (dict(variant=2, lam=math.inf), M.EINVAL),
    (dict(d=96), M.EUNSUPPORTED), (dict(d=32), M.EUNSUPPORTED), (dict(d=256), M.EUNSUPPORTED),
    (dict(d=127, variant=2, lam=0.5), M.EUNSUPPORTED),
    (dict(q=P[0] + 8), M.EINVAL),                   # not 16-byte aligned
    (dict(o=P[3] + 2), M.EINVAL),
    (dict(o=P[0]), M.EINVAL),                       # out aliases q
    (dict(o=P[2] + 64), M.EINVAL),                  # out overlaps v
    (dict(B=2**20, H=2**20, L=2**20, d=128), M.EINVAL),  # byte size overflows
    (dict(B=4096, H=4096, L=65536, d=64), M.EUNSUPPORTED),   # grid too large
    (dict(B=1, H=1, L=2**23, d=128), M.EUNSUPPORTED),        # one head slice = 2 GiB (bf16)
]


@pytest.mark.parametrize("kw,code", BAD)
@pytest.mark.parametrize("f32", [False, True])
def test_invalid_arguments_rejected_before_launch(lib, kw, code, f32):
    assert _call(lib, f32=f32, **kw) == code


def _call_gqa(lib, q=P[0], k=P[1], v=P[2], o=P[3], stream=None, **kw):
    a = dict(OK_ARGS)
    a.setdefault("Hkv", None)
    a.update(kw)
    hkv = a["H"] if a["Hkv"] is None else a["Hkv"]
    return lib.mixer_prefill_gqa_async(q, k, v, o, a["variant"], a["window"],
                                       ctypes.c_float(a["lam"]), a["B"], a["H"], hkv, a["L"],
                                       a["d"], stream)


@pytest.mark.parametrize("kw,code", BAD)
def test_gqa_entry_rejects_what_the_plain_entry_rejects(lib, kw, code):
    # With Hkv = H the grouped entry point is the plain one.
    assert _call_gqa(lib, **kw) == code


@pytest.mark.parametrize("kw", [
    dict(H=4, Hkv=0), dict(H=4, Hkv=-2), dict(H=4, Hkv=3), dict(H=2, Hkv=4),
    dict(H=6, Hkv=4),
])
def test_gqa_rejects_kv_heads_that_do_not_divide_the_heads(lib, kw):
    assert _call_gqa(lib, **kw) == M.EINVAL


def test_gqa_overlap_uses_the_smaller_kv_extent(lib):
    # H=4, Hkv=1, L=64, d=128 bf16: k spans 16 KiB. out starting 16 bytes before its end
    # overlaps k; q and v are far away.
    kv_bytes = 1 * 64 * 128 * 2
    assert _call_gqa(lib, H=4, Hkv=1, o=P[1] + kv_bytes - 16) == M.EINVAL
    assert _call_gqa(lib, H=4, Hkv=1, o=P[2] + kv_bytes - 16) == M.EINVAL


def test_ignored_arguments_do_not_fail_validation_order(lib):
    # window is ignored for FULL and lambda for SLIDING: their bad values must not matter,
    # so these calls reach the next check (null out) and report EINVAL for that.
    assert _call(lib, o=None, variant=0, window=-7) == M.EINVAL
    assert _call(lib, o=None, variant=1, window=4, lam=math.nan) == M.EINVAL


def test_default_stream_entry_validates(lib):
    assert lib.mixer_prefill(None, P[1], P[2], P[3], 0, 0, ctypes.c_float(0), 1, 1, 8, 64) \
        == M.EINVAL


# --------------------------------------------------------------------- scheduler (host)

def test_latin_build_matches_oracle(lib):
    for n in range(1, 12):
        base = [7 * i + 3 for i in range(n)]
        assert M.mixer_latin_build(base) == latin.cyclic_square(base)


def test_table7_schedules(lib):
    code = {"S": 1, "G": 2, "M": 3, "F": 0}
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, expect, *groups = line.split()
            seq = [code[c] for c in "".join(groups)]
            assert M.mixer_latin_check(4, seq) is (expect == "1"), name
    assert M.mixer_latin_build([1, 2, 3, 0]) == [code[c] for c in "SGMFGMFSMFSGFSGM"]


def test_latin_check_agrees_with_oracle_on_every_3x3_grid(lib):
    for g in itertools.product(range(3), repeat=9):
        assert M.mixer_latin_check(3, g) is latin.is_latin(3, list(g))


def test_latin_check_agrees_with_oracle_on_4x4_row_permutations(lib):
    perms = list(itertools.permutations(range(4)))
    count = 0
    for rows in itertools.product(perms, repeat=4):
        sched = [x for r in rows for x in r]
        ok = M.mixer_latin_check(4, sched)
        assert ok is latin.is_latin(4, sched)
        count += ok
    assert count == 576


def test_latin_errors(lib):
    assert lib.mixer_latin_check(0, (ctypes.c_int * 1)(0)) == M.EINVAL
    assert lib.mixer_latin_check(2, None) == M.EINVAL
    assert lib.mixer_latin_build(0, (ctypes.c_int * 1)(0), (ctypes.c_int * 1)()) == M.EINVAL
    assert lib.mixer_latin_build(3, None, (ctypes.c_int * 9)()) == M.EINVAL


def _stack(lib, sched, n=3, ptrs=None, **kw):
    m = n * n
    base = ptrs or [0x1000000 * (i + 1) for i in range(4 * m)]
    arr = lambda off: (ctypes.c_void_p * m)(*base[off * m:(off + 1) * m])  # noqa: E731
    a = dict(window=1024, lam=0.8, B=1, H=2, L=64, d=128)
    a.update(kw)
    return lib.mixer_stack_prefill(n, (ctypes.c_int * m)(*sched), arr(0), arr(1), arr(2),
                                   arr(3), a["window"], ctypes.c_float(a["lam"]), a["B"],
                                   a["H"], a["L"], a["d"], None, None)


def _layers_call(lib, variants, ptrs=None, **kw):
    m = len(variants)
    base = ptrs or [0x1000000 * (i + 1) for i in range(4 * max(m, 1))]
    arr = lambda off: (ctypes.c_void_p * max(m, 1))(*base[off * m:(off + 1) * m])  # noqa: E731
    a = dict(window=1024, lam=0.8, B=1, H=2, L=64, d=128)
    a.update(kw)
    return lib.mixer_layers_prefill(m, (ctypes.c_int * max(m, 1))(*variants), arr(0), arr(1),
                                    arr(2), arr(3), a["window"], ctypes.c_float(a["lam"]),
                                    a["B"], a["H"], a["L"], a["d"], None, None)


def test_layers_runner_validates_every_layer_before_launch(lib):
    # The general runner takes any order (no Latin check) but every layer's arguments are
    # checked before anything is launched.
    assert _layers_call(lib, []) == M.EINVAL                                  # n = 0
    assert lib.mixer_layers_prefill(3, None, None, None, None, None, 0, ctypes.c_float(0),
                                    1, 1, 8, 64, None, None) == M.EINVAL
    assert _layers_call(lib, [0, 0, 0, 1, 1, 1, 2, 2, 3]) == M.EINVAL         # variant 3
    assert _layers_call(lib, [0, 1, 2] * 3, window=0) == M.EINVAL             # sliding layers
    assert _layers_call(lib, [0] * 8 + [2], lam=math.nan) == M.EINVAL         # differential
    ptrs = [0x1000000 * (i + 1) for i in range(36)]
    ptrs[27 + 7] = ptrs[7]                                                     # out[7] = q[7]
    assert _layers_call(lib, [0] * 9, ptrs=ptrs) == M.EINVAL
    assert _layers_call(lib, [0] * 9, d=96) == M.EUNSUPPORTED


def test_stack_rejects_non_latin_before_launch(lib):
    assert _stack(lib, [0, 1, 2, 0, 1, 2, 0, 1, 2]) == M.ENOTLATIN       # periodic
    assert _stack(lib, [0, 0, 0, 1, 1, 1, 2, 2, 2]) == M.ENOTLATIN       # block
    assert _stack(lib, [0] * 9) == M.ENOTLATIN                           # homogeneous


def test_stack_validates_every_layer_before_launch(lib):
    sched = latin.cyclic_square([0, 1, 2])
    assert _stack(lib, sched, window=0) == M.EINVAL                      # sliding layers
    assert _stack(lib, sched, lam=math.nan) == M.EINVAL                  # differential
    assert _stack(lib, sched, d=96) == M.EUNSUPPORTED
    assert _stack(lib, [0, 1, 3, 1, 3, 0, 3, 0, 1]) == M.EINVAL           # variant 3
    ptrs = [0x1000000 * (i + 1) for i in range(36)]
    ptrs[35] = None                                                      # last out is null
    assert _stack(lib, sched, ptrs=ptrs) == M.EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(M.MixerError):
        M.lib()


# ------------------------------------------------ the matrix-core ceiling measurement aid

CEIL_OK = dict(frags=0x10000000, nsets=4, sink=0x20000000, blocks=8, iters=16)
CEIL_BAD = [
    dict(frags=None), dict(sink=None), dict(frags=0x10000008), dict(sink=0x20000004),
    dict(nsets=0), dict(nsets=-1), dict(nsets=(1 << 20) + 1), dict(blocks=0),
    dict(blocks=(1 << 20) + 1), dict(iters=0), dict(iters=6), dict(iters=-4),
    # sink (8 workgroups = 512 KiB) starting inside the fragment sets (32 KiB)
    dict(sink=0x10000000 + 16 * 1024),
    # fragment sets starting inside the sink
    dict(frags=0x20000000 + 500 * 1024),
]


@pytest.mark.parametrize("bad", CEIL_BAD)
def test_ceiling_rejects_bad_arguments(lib, bad):
    a = dict(CEIL_OK)
    a.update(bad)
    rc = lib.mixer_mfma_ceiling_async(a["frags"], a["nsets"], a["sink"], a["blocks"],
                                      a["iters"], None)
    assert rc == M.EINVAL, bad



def test_binding_rejects_an_empty_layer_list():
    with pytest.raises(M.MixerError) as e:
        M.mixer_layers_prefill([], [], [], [], [])
    assert e.value.status == M.EINVAL
