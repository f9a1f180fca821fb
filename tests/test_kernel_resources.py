"""Resource use of every kernel in pa_kernels.hip, from the compiler's own
code-object metadata (device-only assembly for gfx950, the same flags as the
library build): no kernel may use scratch (register spills or private
arrays), and each must fit the 160 KB of LDS a gfx950 compute unit has.
A spill slips in silently when a kernel's register allocation tips over its
budget, and costs far more than its instruction count suggests."""
import os
import re
import subprocess
import tempfile

import pytest

from paged_kv_gqa_attention_amd import build as B

LDS_BYTES = 160 * 1024


@pytest.fixture(scope="module")
def kernels():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = ["hipcc", "-x", "hip"] + B.DEVICE + B.COMMON + \
            ["--cuda-device-only", "-S", os.path.join(B.CSRC, "pa_kernels.hip"), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        text = open(out).read()
    meta = text[text.index("amdhsa.kernels:"):]
    found = {}
    for blk in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name:
            continue
        fields = {k: int(v) for k, v in re.findall(
            r"\.(private_segment_fixed_size|group_segment_fixed_size|vgpr_count|agpr_count):\s+(\d+)", blk)}
        found[name.group(1)] = fields
    assert found, "no kernels in the metadata"
    return found


def test_every_kernel_is_listed(kernels):
    for needle in ("attn_kernel", "mla_hs_kernel", "merge_kernel", "merge_balanced_kernel",
                   "append_kernel", "queue_setup_kernel", "check_kernel"):
        assert any(needle in k for k in kernels), needle


def test_no_kernel_uses_scratch(kernels):
    bad = {k: v["private_segment_fixed_size"] for k, v in kernels.items() if v["private_segment_fixed_size"]}
    assert not bad, bad


def test_every_kernel_fits_lds(kernels):
    bad = {k: v["group_segment_fixed_size"] for k, v in kernels.items() if v["group_segment_fixed_size"] > LDS_BYTES}
    assert not bad, bad
