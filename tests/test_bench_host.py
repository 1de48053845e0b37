"""Host-side logic of bench.py, on the CPU: the useful-work count behind every TFLOP/s figure,
the HBM traffic summary (counter scaling and the source hash that keys it) and the one-GPU
guard. Nothing here touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _pairs_by_enumeration(variant, L, W):
    n = 0
    for i in range(L):
        for j in range(i + 1):
            if variant != "sliding" or i - j <= W - 1:
                n += 1
    return n


@pytest.mark.parametrize("variant,L,W", [
    ("full", 1, 0), ("full", 37, 0), ("full", 128, 0),
    ("sliding", 1, 1), ("sliding", 37, 1), ("sliding", 37, 5), ("sliding", 64, 63),
    ("sliding", 64, 64), ("sliding", 64, 500), ("differential", 50, 0)])
def test_visible_pairs_match_enumeration(variant, L, W):
    # The visibility rule itself (key j visible to query i iff j <= i, and i - j <= W - 1 for
    # the window) counted pair by pair.
    assert bench.visible_pairs(variant, L, W) == _pairs_by_enumeration(variant, L, W)


def test_useful_flops_of_the_stack_workload():
    # B=1, H=16, L=8192, d=128: 4*d flops per visible pair; window 1024 for sliding.
    full = bench.useful_flops("full", 1, 16, 8192, 128, 0)
    sliding = bench.useful_flops("sliding", 1, 16, 8192, 128, 1024)
    diff = bench.useful_flops("differential", 1, 16, 8192, 128, 0)
    assert full == 4 * 128 * 16 * (8192 * 8193 // 2) == diff
    assert sliding == 4 * 128 * 16 * (1024 * 1025 // 2 + (8192 - 1024) * 1024)
    # Three layers of each variant per step of the 3x3 square.
    assert 3 * (full + sliding + diff) == pytest.approx(1.84275e12, rel=1e-5)
    assert bench.executed_per_useful("differential") == 1.5
    assert bench.executed_per_useful("full") == bench.executed_per_useful("sliding") == 1.0


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {\n  // the sum\n  return x + 1; /* one\n more */\n}\n"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("return x + 2;") != bench._code_only("return x + 1;")


def _counter_csv(path, counter, values):
    with open(path, "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for name, kib in values:
            f.write(f'"{name}","{counter}",{kib}\n')


def test_write_traffic_scales_by_the_copy_and_reads_back(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm_traffic.txt"))
    mib = 1024  # KiB
    # The copy kernel reads 256 MiB but the fetch counter shows half of it: fetch scale 2.
    fetch = [("__amd_rocclr_copyBuffer", 128 * mib),
             ("_ZN5mixer3dma18prefill_dma_kernelILi128ELi0EEEvPKDF16b", 60 * mib),
             ("_ZN5mixer3dma18prefill_dma_kernelILi128ELi0EEEvPKDF16b", 70 * mib),
             ("_ZN5mixer3dma19prefill_diff_kernelILi128EEEvPKDF16b", 100 * mib)]
    write = [("__amd_rocclr_copyBuffer", 256 * mib),
             ("_ZN5mixer3dma18prefill_dma_kernelILi128ELi0EEEvPKDF16b", 32 * mib),
             ("_ZN5mixer3dma18prefill_dma_kernelILi128ELi0EEEvPKDF16b", 32 * mib),
             ("_ZN5mixer3dma19prefill_diff_kernelILi128EEEvPKDF16b", 32 * mib)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "test")
    MiB = 1024 * 1024
    # full: mean fetch 65 MiB x 2 + mean write 32 MiB x 1.
    assert bench.read_traffic("full") == pytest.approx((2 * 65 + 32) * MiB)
    assert bench.read_traffic("differential") == pytest.approx((2 * 100 + 32) * MiB)
    assert bench.read_traffic("sliding") is None  # no counters for it


def test_traffic_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    path = tmp_path / "hbm_traffic.txt"
    path.write_text("kernel_source_sha256_16 = 0000000000000000\n"
                    "full_hbm_bytes_per_launch = 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.read_traffic("full") is None
    path.write_text(f"kernel_source_sha256_16 = {bench.kernel_source_hash()}\n"
                    "full_hbm_bytes_per_launch = 123\n")
    assert bench.read_traffic("full") == 123.0


def test_committed_traffic_summary_matches_the_kernel_source():
    # The committed counter summary must describe the kernel as it is now.
    for v in bench.VARIANT_NAMES:
        t = bench.read_traffic(v)
        assert t is not None and t > 4 * 16 * 8192 * 128 * 2  # above the algorithmic bytes


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
