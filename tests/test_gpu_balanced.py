"""GPU parity of balanced decode (plan num_splits = -1) against the oracle:
random batches element by element (bf16/fp8, every head dim, GQA up to 32,
softcap), grids of a few workgroups (every item cut into many pieces) and of
more workgroups than work, empty sequences, sequences without a query token,
and the full-size decode workloads on sampled rows."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def run_balanced(w, num_cus=0, ref=None, rows=None):
    pa = PagedAttention(w, num_splits=-1, num_cus=num_cus)
    print("case", w.name, "balanced W", pa.info.balanced_workgroups, "cus", num_cus, flush=True)
    assert pa.info.balanced_workgroups > 0
    x = DeviceInputs(w)
    out, lse = pa.run("decode", x)
    torch.cuda.synchronize()
    if ref is None:
        ref = H.run_oracle(w, rows=rows)
    return check(w, out, lse, ref[0], ref[1], rows=rows,
                 what="%s/balanced/W%d" % (w.name, pa.info.balanced_workgroups))


@pytest.mark.parametrize("seed", range(12))
def test_balanced_random_decode(seed):
    kv = "fp8_e4m3" if seed % 2 else "bf16"
    rng = np.random.default_rng(900 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    w = H.random_workload(900 + seed, kv_dtype=kv, decode=True, max_len=3000, G=G,
                          Hkv=int(rng.choice([1, 2, 3])), B=int(rng.integers(1, 12)))
    if seed % 4 == 3:
        w.softcap = 1.5
    ref = H.run_oracle(w)
    for cus in (0, 1, 3, 7):
        run_balanced(w, num_cus=cus, ref=ref)


def test_balanced_empty_and_queryless_sequences():
    # lengths 0, 1, 3, 129 and long ones; decode rows given through cu_q_lens,
    # three sequences without a query token this step (one of them empty)
    L = [0, 1, 129, 2000, 3, 700, 128]
    ql = [0, 1, 0, 1, 1, 0, 1]
    w = synth.build(name="edge_balanced", seq_lens=L, q_lens=ql, num_q_heads=8, num_kv_heads=2,
                    head_dim=128, page_size=16, seed=31, threads=1)
    ref = H.run_oracle(w)
    for cus in (0, 1, 2, 5):
        run_balanced(w, num_cus=cus, ref=ref)


def test_balanced_one_long_sequence_over_many_workgroups():
    w = synth.build(name="one_long", seq_lens=[30000], q_lens=[1], num_q_heads=64, num_kv_heads=2,
                    head_dim=256, page_size=128, seed=32, kv_dtype="fp8_e4m3", threads=4)
    ref = H.run_oracle(w)
    run_balanced(w, ref=ref)
    run_balanced(w, num_cus=9, ref=ref)


@pytest.mark.slow
def test_balanced_full_size():
    for make in (synth.decode_llama8b, synth.decode_fp8_long):
        w = make()
        rows = synth.sample_rows(w, per_seq=3, heads=8)
        run_balanced(w, rows=rows)
