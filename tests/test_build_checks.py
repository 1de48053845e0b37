"""The build's resource check, on the CPU: the bf16 kernel file's key loops wait on their own
untracked tile loads with counted waits, so its kernels must build with no vector-register
spills and no scratch (a spill to scratch is a counted memory access). Scalar registers
spilled to lanes of a vector register are register moves and pass. build.py reads the
compiler's resource remarks for that file and refuses to link a library that breaks this."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from heterogeneous_attention_mixer_amd import build  # noqa: E402

REMARKS = """\
a.hip:10:1: remark: Function Name: _Z2k1v [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     VGPRs: 250 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:10:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark: Function Name: _Z2k2v [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     ScratchSize [bytes/lane]: 28 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:20:1: remark:     VGPRs Spill: 6 [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark: Function Name: _Z2k3v [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark:     SGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
a.hip:30:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
a.hip:40:1: remark: Function Name: _Z2k4v [-Rpass-analysis=kernel-resource-usage]
a.hip:40:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]
a.hip:40:1: remark:     SGPRs Spill: 40 [-Rpass-analysis=kernel-resource-usage]
a.hip:40:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spilling_kernels_are_named():
    bad = build.spilling_kernels(REMARKS)
    assert ("_Z2k2v", "VGPRs Spill 6") in bad
    assert ("_Z2k2v", "ScratchSize [bytes/lane] 28") in bad
    assert ("_Z2k4v", "ScratchSize [bytes/lane] 8") in bad
    # scalar spills with no scratch live in vector-register lanes: no memory access
    assert not [k for k, _ in bad if k in ("_Z2k1v", "_Z2k3v")]


def test_the_checked_file_is_the_bf16_kernel():
    assert "attn_prefill_dma.hip" in build.NO_SPILL
    assert any(s.endswith("attn_prefill_dma.hip") for s in build.SOURCES)
