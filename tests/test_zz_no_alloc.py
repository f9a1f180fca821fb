"""pa_run_decode_static (the allocation-free decode entry point) against
pa_run_decode with a caller workspace: same plan, same inputs, outputs equal
bit for bit and within the oracle tolerance, on two calls in a row whose
second input is smaller than the first (the static scratch keeps the first
call's contents).  Both a balanced plan (records and schedule words in the
scratch) and a split plan (partials in the scratch) are covered."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import binding as B
from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def both_entries(w, num_splits):
    pa = PagedAttention(w, num_splits=num_splits)
    ws = B.pa_workspace_bytes(pa.plan)
    print("case", w.name, "splits", num_splits, "workspace", ws, flush=True)
    assert 0 < ws <= B.PA_STATIC_SCRATCH_BYTES
    x = DeviceInputs(w)
    ref_out, ref_lse = pa.run("decode", x)
    out, lse = pa.new_outputs(x)
    out.fill_(7.0)
    lse.fill_(7.0)
    a = pa.args(x, out, lse, workspace=None)
    a.workspace = None          # ignored by the static entry point
    a.workspace_bytes = 0
    B.pa_run_decode_static(pa.plan, a, B.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), w.name + ": O differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), w.name + ": LSE differs"
    ro, rl = H.run_oracle(w)
    check(w, out, lse, ro, rl, what=w.name + "/static")


@pytest.mark.parametrize("num_splits", [-1, 3])
def test_static_decode_matches_workspace_decode(num_splits):
    big = synth.build(name="static_big", seq_lens=[3000, 17, 1200, 2500, 640, 4095],
                      q_lens=[1] * 6, num_q_heads=64, num_kv_heads=2, head_dim=256,
                      page_size=128, seed=41, kv_dtype="fp8_e4m3", threads=4)
    small = synth.build(name="static_small", seq_lens=[900, 33, 2048], q_lens=[1] * 3,
                        num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, seed=42,
                        threads=4)
    both_entries(big, num_splits)
    both_entries(small, num_splits)


def test_static_decode_rejects_plans_beyond_the_scratch():
    # 4 splits of 4096 rows x 64 heads x 256 floats exceed the 32 MiB array
    w = synth.build(name="static_huge", seq_lens=[8192] * 4, q_lens=[1] * 4, num_q_heads=64,
                    num_kv_heads=2, head_dim=256, page_size=128, seed=43, kv_dtype="fp8_e4m3",
                    threads=4)
    pa = PagedAttention(w, num_splits=4, max_total_q=4096)
    assert B.pa_workspace_bytes(pa.plan) > B.PA_STATIC_SCRATCH_BYTES
    x = DeviceInputs(w)
    out, lse = pa.new_outputs(x)
    a = pa.args(x, out, lse)
    with pytest.raises(B.PaError) as e:
        B.pa_run_decode_static(pa.plan, a, B.current_stream())
    assert e.value.code == B.PA_ERR_SCRATCH
