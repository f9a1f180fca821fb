"""GPU parity at full size: the large workloads in the launch configuration
bench.py times (plus the other entry points that accept them), compared with
the oracle element by element.  The decode workloads are checked on every
row; the prefill and the serving mix on rows that touch every work item of
the launch (each q-block, each wave's token slice, each KV head) plus every
sequence's first and last token at every head; other schedules on sampled
rows."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def run_sampled(w, mode, num_splits=0, per_seq=3, heads=4):
    print("case", w.name, mode, "splits", num_splits, flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=num_splits)
    out, lse = pa.run(mode, x)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w, per_seq=per_seq, heads=heads)
    ref = H.run_oracle(w, rows=rows)
    return check(w, out, lse, ref[0], ref[1], rows=rows,
                 what="%s/%s/S%d" % (w.name, mode, pa.info.num_splits))


def run_rows(w, mode, rows, num_splits=0):
    """One run of the bench launch configuration, checked on `rows` (None:
    every row)."""
    print("case", w.name, mode, "splits", num_splits, "rows", "all" if rows is None else len(rows),
          flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=num_splits)
    out, lse = pa.run(mode, x)
    torch.cuda.synchronize()
    ref = H.run_oracle(w, rows=rows)
    return check(w, out, lse, ref[0], ref[1], rows=rows,
                 what="%s/%s/S%d" % (w.name, mode, pa.info.num_splits)), pa


def test_decode_llama8b_full():
    w = synth.decode_llama8b()
    run_rows(w, "decode", None)                   # every row
    run_sampled(w, "decode", num_splits=3)
    run_sampled(w, "mixed")


def test_prefill_causal_full():
    w = synth.prefill_causal()
    pa = PagedAttention(w)
    rows = H.cover_rows(w, pa.info.q_block_tokens)
    assert len(rows) > 30000
    run_rows(w, "prefill", rows)                  # every (q-block, wave slice, KV head)
    run_sampled(w, "mixed", per_seq=6)


def test_prefill_causal_d256_full():
    # head dim 256 (row-split schedule), every (q-block, wave slice, KV head)
    w = synth.prefill_causal_d256()
    pa = PagedAttention(w)
    rows = H.cover_rows(w, pa.info.q_block_tokens)
    run_rows(w, "prefill", rows)
    run_sampled(w, "mixed", per_seq=4)


def test_mixed_24b_full():
    w = synth.mixed_24b()
    pa = PagedAttention(w)
    rows = H.cover_rows(w, pa.info.mixed_q_block_tokens)
    run_rows(w, "mixed", rows)                    # every queue item, every decode row
    run_sampled(w, "prefill", per_seq=4)
    ws = synth.mixed_24b(shuffle=True)
    run_rows(ws, "mixed", H.cover_rows(ws, pa.info.mixed_q_block_tokens))


def test_decode_fp8_long_full():
    w = synth.decode_fp8_long()
    run_rows(w, "decode", None)                   # every row (balanced schedule)
    run_sampled(w, "decode", num_splits=1, heads=8)
    run_sampled(w, "mixed", heads=8)


def test_full_size_outputs_are_finite_everywhere():
    # every row, not just the sample: poisoned tails never leak
    for make, mode in ((synth.decode_llama8b, "decode"), (synth.decode_fp8_long, "decode"),
                       (synth.mixed_24b, "mixed"), (synth.prefill_causal, "prefill"),
                       (synth.prefill_causal_d256, "prefill")):
        w = make()
        x = DeviceInputs(w)
        pa = PagedAttention(w)
        out, lse = pa.run(mode, x)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out.float()).all()), w.name
        assert bool(torch.isfinite(lse).all()), w.name


def test_large_batches_span_wide_grids():
    # 6,000 short decode rows (a grid of 6,000 x 8 workgroups; plain,
    # balanced and mixed) and a mixed batch of about 36,000 tokens (12 long
    # prefills, 12 decode rows; over 1,000 q-blocks per KV head), checked on
    # sampled rows
    rng = np.random.default_rng(77)
    L = rng.integers(1, 200, size=6000)
    w = synth.build(name="decode_6000", seq_lens=L, q_lens=np.ones(6000, dtype=np.int64),
                    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, seed=78)
    run_sampled(w, "decode", per_seq=1, heads=2)
    run_sampled(w, "decode", num_splits=-1, per_seq=1, heads=2)
    run_sampled(w, "mixed", per_seq=1, heads=2)
    L = rng.integers(2000, 4000, size=24)
    q = np.where(np.arange(24) % 2 == 0, L, 1)
    w = synth.build(name="mixed_36k", seq_lens=L, q_lens=q, num_q_heads=16, num_kv_heads=4,
                    head_dim=64, page_size=32, seed=79)
    run_sampled(w, "mixed", per_seq=3, heads=2)
    run_sampled(w, "prefill", per_seq=3, heads=2)
