"""Host-side logic of bench.py, on the CPU: the useful-work count behind every TFLOP/s figure,
the executed matrix-instruction count of the kernels' tile schedule, the counter summaries
(HBM traffic, matrix-pipe busy share; counter scaling and the source hash that keys them)
and the one-GPU guard. Nothing here touches a GPU."""
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


def test_executed_mfmas_closed_forms():
    # Full at B=1, H=16, L=4096 on the pipelined kernel (32 query tiles of 128 rows, one
    # wave per row block; 256 tiles of 256 rows would be one per CU): query tile t spans key
    # tiles 0..2t+1, and each of its 4 waves issues 32 MFMAs per tile (scores 16 + value
    # product 16, the first iteration's value product on zeros standing in for the one
    # before the first tile); the last tile's value product after the loop adds 16 for the
    # waves of the last 64 rows, the only ones that see that tile.
    assert not bench.full_takes_phase_kernel(1, 16, 4096)
    per_head = sum(4 * 32 * (2 * t + 2) + 2 * 16 for t in range(32))
    assert bench.executed_mfmas("full", 1, 16, 4096, 128, 0) == 16 * per_head
    # Full at L=8192 on the phase-separated kernel: 32 query tiles of 256 rows, 8 waves,
    # hi = 4t + 3, hi + 2 matrix phases of 16 + 16 MFMAs, and hi + 1 row-sum passes of 4.
    assert bench.full_takes_phase_kernel(1, 16, 8192)
    per_head = sum(8 * (4 * t + 5) * 32 for t in range(32))
    small = sum(8 * (4 * t + 4) * 4 for t in range(32))
    assert bench.executed_mfma_split("full", 1, 16, 8192, 128, 0) == (16 * per_head,
                                                                       16 * small)
    # Differential: 8 waves, hi + 2 matrix phases of 8 + 16 MFMAs each, hi = 2t + 1, and 4
    # row-sum instructions (16x16x32) per exponential pass, hi + 1 passes.
    per_head = sum(8 * (2 * t + 3) * 24 for t in range(64))
    small = sum(8 * (2 * t + 2) * 4 for t in range(64))
    assert bench.executed_mfma_split("differential", 1, 16, 8192, 128, 0) == (
        16 * per_head, 16 * small)
    assert bench.executed_mfmas("differential", 1, 16, 8192, 128, 0) == 16 * (per_head + small)
    assert bench.executed_flops("differential", 1, 16, 8192, 128, 0) == 16 * (
        per_head * 32768 + small * 16384)
    # Sliding, W = 1024, a query tile past the first window: 18 key tiles, every wave all of
    # them; the waves of rows 64..127 skip the first tile's scores (it lies below their
    # windows) and those of rows 0..63 the last tile's value product (it lies past them).
    full_tiles = 4 * (32 * 18 + 16) - 2 * 16 - 2 * 16
    assert bench.executed_mfmas("sliding", 1, 1, 2048, 128, 1024, n_cu=0) - \
        bench.executed_mfmas("sliding", 1, 1, 1920, 128, 1024, n_cu=0) == full_tiles


def _paired_mfmas_by_simulation(B, H, L, d):
    # The paired key-split loop of the full kernel, wave by wave and iteration by iteration:
    # the prologue's scores, then per iteration the value product of the tile two back and,
    # unless the iteration is the wave's last, the scores of the tile two ahead; a wave's
    # iterations are those of its tiles its rows see (at least its first); the value product
    # of its last tile after the loop if its rows see that tile.
    qk, pv = 2 * (d // 16), 4 * (d // 32)
    nt = (L + 63) // 64
    total = 0
    for p in range(nt // 2):
        th = nt - 1 - p
        n_it = (min(th * 64 + 64, L) - 1) // 64 // 2 + 1
        for rb in range(4):
            first = p * 64 + 32 * rb if rb < 2 else th * 64 + 32 * (rb - 2)
            last_tile = (first + 31) // 64
            for half in range(2):
                its = [it for it in range(n_it) if 2 * it + half <= last_tile] or [0]
                n = qk if (half == 0 or 64 * half <= first + 31) else 0
                for it in its:
                    n += pv + (qk if it != its[-1] else 0)
                if (2 * its[-1] + half) * 64 <= first + 31:
                    n += pv
                total += n
    return B * H * total


@pytest.mark.parametrize("B,H,L,d", [(1, 16, 2048, 128), (1, 3, 128, 128), (2, 3, 1000, 64),
                                     (1, 1, 1989, 128), (1, 16, 640, 64)])
def test_executed_mfmas_of_paired_tiles(B, H, L, d):
    assert B * H * ((L + 127) // 128) <= 256 and ((L + 63) // 64) % 2 == 0
    assert bench.executed_mfmas("full", B, H, L, d, 0) == _paired_mfmas_by_simulation(B, H, L, d)


@pytest.mark.parametrize("variant,L,W", [("full", 1, 0), ("full", 300, 0), ("full", 2048, 0),
                                         ("sliding", 777, 100), ("sliding", 8192, 1024),
                                         ("differential", 129, 0), ("differential", 4096, 0)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_cu", [0, 256])
def test_executed_mfmas_cover_the_useful_work(variant, L, W, d, n_cu):
    # Whole tiles and masked keys: never less matrix work than the useful flops, and the
    # differential's second value product makes it at least 1.5 times the useful work.
    ex = bench.executed_flops(variant, 1, 4, L, d, W, n_cu=n_cu)
    fl = bench.useful_flops(variant, 1, 4, L, d, W)
    assert ex >= (1.5 if variant == "differential" else 1.0) * fl


def test_executed_mfmas_match_the_committed_counters():
    # The instruction counter of the committed SQ summary (taken on the bench's stack) is
    # the same count, exactly, while the summary describes the current kernel source.
    for v in bench.VARIANT_NAMES:
        sq = bench.read_sq(v)
        if sq is None:
            pytest.skip("no SQ summary for the current kernel source")
        w = 1024 if v == "sliding" else 0
        assert sq["sq_insts_mfma"] == bench.executed_mfmas(v, 1, 16, 8192, 128, w)


def test_executed_mfmas_match_the_counters_at_every_bench_length():
    # SQ_INSTS_MFMA of one profiled run over the stack and the sweep points (full at 2K, 8K
    # and 32K, including the paired key split at 2K; the differential at 8K and 32K; sliding
    # at 8K), committed with the kernel source hash it was taken on.
    path = os.path.join(ROOT, "profiles", "mfma_counts_by_length.txt")
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != bench.kernel_source_hash():
        pytest.skip("the counts were taken on another kernel source")
    for variant, L in (("full", 2048), ("full", 8192), ("full", 32768), ("sliding", 8192),
                       ("differential", 8192), ("differential", 32768)):
        w = 1024 if variant == "sliding" else 0
        assert int(kv[f"{variant}_L{L}_sq_insts_mfma"]) == \
            bench.executed_mfmas(variant, 1, 16, L, 128, w), (variant, L)


def test_write_sq_reads_busy_share_and_clock(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SQ_FILE", str(tmp_path / "sq_busy.txt"))
    path = tmp_path / "c.csv"
    name = "_ZN5mixer3dma20prefill_phase_kernelILi128ELi0EEEvPKDF16b"
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value",'
                '"Start_Timestamp","End_Timestamp"\n')
        for did, busy, grbm in ((1, 1024 * 500, 8 * 1000), (2, 1024 * 600, 8 * 1000)):
            for cn, cv in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_INSTS_MFMA", 77),
                           ("GRBM_GUI_ACTIVE", grbm)):
                f.write(f'{did},"{name}","{cn}",{cv},1000,1500\n')
    bench.write_sq(str(path), "test")
    sq = bench.read_sq("full")
    assert sq["mfma_busy"] == pytest.approx(0.55)        # (500 + 600) / 2 / 1000
    assert sq["sq_insts_mfma"] == 77
    assert sq["effective_clock_ghz"] == pytest.approx(2.0)  # 1000 cycles in 500 ns
    assert bench.read_sq("sliding") is None


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


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
    full = "_ZN5mixer3dma20prefill_phase_kernelILi128ELi0EEEvPKDF16b"
    diff = "_ZN5mixer3dma20prefill_phase_kernelILi128ELi2EEEvPKDF16b"
    fetch = [("__amd_rocclr_copyBuffer", 128 * mib), (full, 60 * mib), (full, 70 * mib),
             (diff, 100 * mib)]
    write = [("__amd_rocclr_copyBuffer", 256 * mib), (full, 32 * mib), (full, 32 * mib),
             (diff, 32 * mib)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "test")
    MiB = 1024 * 1024
    # full: mean fetch 65 MiB x 2 + mean write 32 MiB x 1.
    assert bench.read_traffic("full") == pytest.approx((2 * 65 + 32) * MiB)
    assert bench.read_traffic("differential") == pytest.approx((2 * 100 + 32) * MiB)
    assert bench.read_traffic("sliding") is None  # no counters for it


def test_launch_threads_follow_the_launcher():
    # Pipelined kernel: 128-row query tiles, 4 waves per full/sliding workgroup, 8 with the
    # key split (at most one workgroup per CU). Phase-separated kernel (the differential's
    # 128-row units; full's 256-row units on grids of more of them than CUs): 8 waves per
    # unit, or one workgroup per CU (persistent) when there are more units than CUs. The
    # profiler reported these Grid_Size values for the bench's launches.
    assert bench.launch_threads("full", 1, 16, 8192) == 256 * 512         # persistent
    assert bench.launch_threads("sliding", 1, 16, 8192) == 262144
    assert bench.launch_threads("differential", 1, 16, 8192) == 256 * 512  # persistent
    assert bench.launch_threads("full", 1, 16, 2048) == 131072       # key split
    assert bench.launch_threads("full", 1, 16, 4096) == 512 * 256    # pipelined
    assert bench.launch_threads("full", 1, 16, 32768) == 256 * 512
    assert bench.launch_threads("differential", 1, 16, 32768) == 256 * 512
    assert bench.launch_threads("differential", 1, 16, 2048) == 256 * 512  # one per unit
    assert bench.launch_threads("differential", 1, 2, 2048) == 32 * 512
    assert bench.launch_threads("full", 1, 1, 300) == 3 * 512
    assert bench.launch_threads("full", 2, 80, 333) == 256 * 512


def test_counter_summaries_take_the_stack_launches_only(tmp_path, monkeypatch):
    # A run that also times other lengths: launches of the same kernel with another grid
    # stay out of the per-launch averages.
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm_traffic.txt"))
    monkeypatch.setattr(bench, "SQ_FILE", str(tmp_path / "sq_busy.txt"))
    name = "_ZN5mixer3dma17prefill_dma_kernelILi128ELi1ELi1EEEvPKDF16b"
    stack, other = bench.launch_threads("sliding", 1, 16, 8192), bench.launch_threads(
        "sliding", 1, 16, 32768)
    mib = 1024
    for counter, copy_kib, kib in (("FETCH_SIZE", 256 * mib, (10 * mib, 999 * mib)),
                                   ("WRITE_SIZE", 256 * mib, (4 * mib, 99 * mib))):
        with open(tmp_path / f"{counter}.csv", "w") as f:
            f.write('"Dispatch_Id","Grid_Size","Kernel_Name","Counter_Name","Counter_Value"\n')
            f.write(f'1,131072,"__amd_rocclr_copyBuffer","{counter}",{copy_kib}\n')
            f.write(f'2,{stack},"{name}","{counter}",{kib[0]}\n')
            f.write(f'3,{other},"{name}","{counter}",{kib[1]}\n')
    bench.write_traffic(str(tmp_path / "FETCH_SIZE.csv"), str(tmp_path / "WRITE_SIZE.csv"),
                        "test")
    assert bench.read_traffic("sliding") == pytest.approx(14 * 1024 * 1024)
    with open(tmp_path / "sq.csv", "w") as f:
        f.write('"Dispatch_Id","Grid_Size","Kernel_Name","Counter_Name","Counter_Value",'
                '"Start_Timestamp","End_Timestamp"\n')
        for did, grid, busy in ((1, stack, 1024 * 500), (2, other, 1024 * 900)):
            for cn, cv in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_INSTS_MFMA", did),
                           ("GRBM_GUI_ACTIVE", 8 * 1000)):
                f.write(f'{did},{grid},"{name}","{cn}",{cv},1000,1500\n')
    bench.write_sq(str(tmp_path / "sq.csv"), "test")
    sq = bench.read_sq("sliding")
    assert sq["mfma_busy"] == pytest.approx(0.5) and sq["sq_insts_mfma"] == 1


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
