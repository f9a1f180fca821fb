"""GPU parity of the task-queue schedule of mixed batches (plan num_splits =
-1): persistent workgroups draw prefill-type and decode-type items from two
queues laid out by a setup launch.  Random batches (all head dims, bf16 and
fp8, causal or not, soft-capped), few workgroups for many items, more than
1024 sequences (the setup scan's chunked path), empty sequences, the
full-size serving mix in both orders on sampled rows, and graph replays with
the query lengths rewritten in place, all against the oracle."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_full import run_sampled
from tests.test_gpu_graph import _capture
from tests.test_gpu_parity import check, run_and_check

pytestmark = pytest.mark.gpu


def run_queue(w, num_cus=0, ref=None, rows=None):
    print("case", w.name, "mixed queue cus", num_cus, flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=-1, num_cus=num_cus)
    assert pa.info.queue_workgroups > 0
    out, lse = pa.run("mixed", x)
    torch.cuda.synchronize()
    if ref is None:
        ref = H.run_oracle(w, rows=rows)
    return check(w, out, lse, ref[0], ref[1], rows=rows, what="%s/queue" % w.name)


@pytest.mark.parametrize("seed", range(14))
def test_queue_random(seed):
    kv = "fp8_e4m3" if seed % 3 == 2 else "bf16"
    rng = np.random.default_rng(1100 + seed)
    w = H.random_workload(1100 + seed, kv_dtype=kv, causal=(seed % 5 != 4), max_len=300,
                          G=int(rng.choice([1, 2, 4, 8, 16, 32])), Hkv=int(rng.choice([1, 2, 3])),
                          B=int(rng.integers(1, 12)))
    if seed % 4 == 1:
        w.softcap = 2.0
    ref = H.run_oracle(w)
    run_queue(w, ref=ref)
    run_queue(w, num_cus=3, ref=ref)          # 6 workgroups drain every item


def test_queue_many_sequences_and_empty_ones():
    # 1500 sequences: decode rows, some chunked-prefill rows, some with no
    # query token at all
    rng = np.random.default_rng(41)
    B_ = 1500
    L = rng.integers(1, 90, size=B_)
    kind = rng.random(B_)
    ql = np.where(kind < 0.1, 0, np.where(kind < 0.9, 1, np.minimum(L, rng.integers(2, 60, size=B_))))
    w = synth.build(name="queue_many", seq_lens=L, q_lens=ql, num_q_heads=8, num_kv_heads=2,
                    head_dim=64, page_size=16, seed=42, threads=4)
    run_queue(w)
    run_and_check(w, "mixed")


def test_queue_full_size():
    run_sampled_queue = lambda w: run_queue(w, rows=synth.sample_rows(w, per_seq=4, heads=4))
    run_sampled_queue(synth.mixed_24b())
    run_sampled_queue(synth.mixed_24b(shuffle=True))
    run_sampled_queue(synth.mixed_24b(kv_dtype="fp8_e4m3"))


def test_graph_replay_queue_with_new_query_lengths():
    # same shapes, different split of the tokens into sequences: the queue
    # lists are rebuilt by the setup launch on every replay
    B_, page, C = 10, 16, 40
    rng = np.random.default_rng(51)
    L = rng.integers(300, C * page - 16, size=B_)
    qa = np.array([1, 1, 200, 1, 1, 60, 1, 1, 1, 33])
    qb = np.array([90, 1, 1, 1, 150, 1, 1, 1, 50, 4])
    assert qa.sum() == qb.sum()
    P = 2 * int(sum((L + page - 1) // page)) + 2
    mk = lambda name, q, sd: synth.build(name=name, seq_lens=L, q_lens=q, num_q_heads=16,
                                         num_kv_heads=4, head_dim=128, page_size=page, seed=sd,
                                         pt_cols=C, num_pages=P, threads=2)
    wa, wb = mk("queueA", qa, 61), mk("queueB", qb, 62)
    x = DeviceInputs(wa)
    pa = PagedAttention(wa, num_splits=-1, num_cus=19)        # wa has the longer query run
    out, lse = pa.new_outputs(x)
    refs = [H.run_oracle(wa), H.run_oracle(wb)]
    pa.run("mixed", x, out=out, lse=lse)
    torch.cuda.synchronize()
    check(wa, out, lse, *refs[0], what="queue eager")
    g = _capture(lambda: pa.run("mixed", x, out=out, lse=lse))
    for rep in range(4):
        w = (wa, wb)[rep % 2]
        for dst, src in ((x.q, w.q), (x.k_pool, w.k_pool), (x.v_pool, w.v_pool),
                         (x.page_table, w.page_table), (x.seq_lens, w.seq_lens),
                         (x.cu_q_lens, w.cu_q_lens)):
            dst.copy_(src)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(w, out, lse, *refs[rep % 2], what="queue replay %d" % rep)
        pa.run("mixed", x, out=out, lse=lse)     # eager work between replays
        torch.cuda.synchronize()
        check(w, out, lse, *refs[rep % 2], what="queue eager %d" % rep)
