"""GPU behaviour around the kernels: HIP-graph capture (split, balanced and MLA
decode, mixed runs, the KV append) with metadata or contents mutated in
place between replays, workspace reuse across calls and plans, a row-strided
page table whose padding columns name the poison page, empty sequences, and
non-causal runs."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import binding as B
from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def twin_workloads(seed, decode):
    """Two workloads with identical shapes (B, T, pool, table width) and
    different lengths, pages and values."""
    rng = np.random.default_rng(seed)
    B_, page, C = 12, 16, 40
    q = np.ones(B_, dtype=np.int64) if decode else rng.integers(1, 40, size=B_)
    L0 = rng.integers(200, C * page - 16, size=B_)
    L1 = rng.integers(200, C * page - 16, size=B_)
    P = int(sum((L0 + page - 1) // page)) + int(sum((L1 + page - 1) // page)) + 2
    mk = lambda name, L, sd: synth.build(name=name, seq_lens=L, q_lens=q, num_q_heads=16,
                                         num_kv_heads=4, head_dim=128, page_size=page, seed=sd,
                                         pt_cols=C, num_pages=P, threads=2)
    return mk("twinA", L0, seed), mk("twinB", L1, seed + 1)


@pytest.mark.parametrize("mode", ["decode", "mixed"])
def test_graph_replay_with_mutated_metadata(mode):
    wa, wb = twin_workloads(7 if mode == "decode" else 8, decode=(mode == "decode"))
    assert wa.q.shape == wb.q.shape and wa.k_pool.shape == wb.k_pool.shape
    x = DeviceInputs(wa)
    pa = PagedAttention(wa, num_splits=3 if mode == "decode" else 0,
                        max_seq_len=max(wa.max_seq_len, wb.max_seq_len))
    out, lse = pa.new_outputs(x)
    ref_a = H.run_oracle(wa)
    ref_b = H.run_oracle(wb)
    # eager first
    pa.run(mode, x, out=out, lse=lse)
    torch.cuda.synchronize()
    check(wa, out, lse, *ref_a, what="eager")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.run(mode, x, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(3):
        w, ref = (wa, ref_a) if rep % 2 == 0 else (wb, ref_b)
        # rewrite metadata and contents in place, then replay
        x.q.copy_(w.q)
        x.k_pool.copy_(w.k_pool)
        x.v_pool.copy_(w.v_pool)
        x.page_table.copy_(w.page_table)
        x.cu_q_lens.copy_(w.cu_q_lens)
        x.seq_lens.copy_(w.seq_lens)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(w, out, lse, *ref, what="replay %d" % rep)


def test_workspace_shared_across_plans_and_calls():
    w1 = H.random_workload(301, decode=True, B=6, D=128, page=16, G=4, Hkv=2, max_len=2000)
    w2 = H.random_workload(302, decode=True, B=3, D=128, page=16, G=4, Hkv=2, max_len=2000)
    x1, x2 = DeviceInputs(w1), DeviceInputs(w2)
    p1 = PagedAttention(w1, num_splits=5)
    p2 = PagedAttention(w2, num_splits=4)
    ws = torch.empty(max(B.pa_workspace_bytes(p1.plan), B.pa_workspace_bytes(p2.plan)),
                     dtype=torch.uint8, device="cuda")
    r1, r2 = H.run_oracle(w1), H.run_oracle(w2)
    for _ in range(2):
        o1, l1 = p1.new_outputs(x1)
        o2, l2 = p2.new_outputs(x2)
        p1.run("decode", x1, out=o1, lse=l1, workspace=ws)
        p2.run("decode", x2, out=o2, lse=l2, workspace=ws)
        torch.cuda.synchronize()
        check(w1, o1, l1, *r1, what="plan1")
        check(w2, o2, l2, *r2, what="plan2")


def test_row_strided_page_table_with_garbage_padding():
    # a [B, 2, C]-style table: the kernels get row stride 2C; the second half of
    # every row names the NaN-filled poison page, so reading it would show up
    base = H.random_workload(303, B=4, D=64, page=32, G=2, Hkv=2, max_len=300)
    C = base.pt_cols
    pt = np.full((base.num_seqs, 2 * C), base.poison_page, dtype=np.int32)
    pt[:, :C] = base.page_table.numpy()
    base.page_table = torch.from_numpy(pt)
    ref = H.run_oracle(base)
    x = DeviceInputs(base)
    pa = PagedAttention(base)
    assert pa.desc.page_table_row_stride == 2 * C and pa.desc.page_table_cols == C
    for mode in ("prefill", "mixed"):
        out, lse = pa.run(mode, x)
        torch.cuda.synchronize()
        check(base, out, lse, *ref, what="strided/" + mode)


def test_empty_sequences_and_zero_length_queries():
    # a sequence with q_len 0 contributes no rows; one with L = 0 and q_len 0 too
    w = synth.build(name="empties", seq_lens=[40, 0, 70, 33], q_lens=[40, 0, 0, 5],
                    num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, seed=5,
                    threads=1)
    ref = H.run_oracle(w)
    x = DeviceInputs(w)
    pa = PagedAttention(w)
    for mode in ("prefill", "mixed"):
        out, lse = pa.run(mode, x)
        torch.cuda.synchronize()
        check(w, out, lse, *ref, what="empties/" + mode)


@pytest.mark.parametrize("seed", range(4))
def test_non_causal(seed):
    w = H.random_workload(400 + seed, causal=False, max_len=200, kv_dtype="bf16" if seed % 2 else "fp8_e4m3")
    ref = H.run_oracle(w)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=2)
    for mode in ("prefill", "mixed"):
        out, lse = pa.run(mode, x)
        torch.cuda.synchronize()
        check(w, out, lse, *ref, what="noncausal/" + mode)


def test_long_window_crosses_page_cache_chunks():
    # more keys than one LDS page-id chunk holds (1024 pages of 16): the kernels
    # refill the cache mid-sequence
    L = [20000, 17000]
    w = synth.build(name="long", seq_lens=L, q_lens=[1, 1], num_q_heads=8, num_kv_heads=2,
                    head_dim=64, page_size=16, seed=11, threads=4)
    ref = H.run_oracle(w)
    x = DeviceInputs(w)
    for S in (1, 2):
        pa = PagedAttention(w, num_splits=S)
        out, lse = pa.run("decode", x)
        torch.cuda.synchronize()
        check(w, out, lse, *ref, what="long/S%d" % S)
    wq = synth.build(name="longq", seq_lens=L, q_lens=[300, 77], num_q_heads=8, num_kv_heads=2,
                     head_dim=64, page_size=16, seed=12, threads=4)
    rows = synth.sample_rows(wq, per_seq=6, heads=8)
    refq = H.run_oracle(wq, rows=rows)
    xq = DeviceInputs(wq)
    pa = PagedAttention(wq)
    for mode in ("prefill", "mixed"):
        out, lse = pa.run(mode, xq)
        torch.cuda.synchronize()
        check(wq, out, lse, *refq, rows=rows, what="longq/" + mode)


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def test_graph_replay_balanced_decode():
    # the balanced schedule rewrites its unit offsets in the workspace on
    # every run; replays with other lengths must see them refreshed
    wa, wb = twin_workloads(17, decode=True)
    x = DeviceInputs(wa)
    pa = PagedAttention(wa, num_splits=-1, num_cus=37,
                        max_seq_len=max(wa.max_seq_len, wb.max_seq_len))
    assert pa.info.balanced_workgroups == 37 * 2
    out, lse = pa.new_outputs(x)
    refs = [H.run_oracle(wa), H.run_oracle(wb)]
    pa.run("decode", x, out=out, lse=lse)
    torch.cuda.synchronize()
    check(wa, out, lse, *refs[0], what="balanced eager")
    g = _capture(lambda: pa.run("decode", x, out=out, lse=lse))
    for rep in range(4):
        w = (wa, wb)[rep % 2]
        for dst, src in ((x.q, w.q), (x.k_pool, w.k_pool), (x.v_pool, w.v_pool),
                         (x.page_table, w.page_table), (x.seq_lens, w.seq_lens)):
            dst.copy_(src)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(w, out, lse, *refs[rep % 2], what="balanced replay %d" % rep)


def test_graph_replay_mla():
    import dataclasses
    import oracle
    from paged_kv_gqa_attention_amd.attention import MlaDecode
    wa = synth.build_mla(name="mla_graph", seq_lens=[700, 90, 1300, 33], num_q_heads=64, page_size=32,
                         seed=41, threads=2)
    qb = synth.normal_bf16(wa.q.numel(), 42, 2, 2).view(wa.q.shape)
    wb = dataclasses.replace(wa, q=qb, seq_lens=torch.tensor([650, 1, 1290, 20], dtype=torch.int32))
    m = MlaDecode(wa, num_splits=3)
    out, lse = m.new_outputs()
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def ref(w):
        return oracle.mla_decode(q_bits=bits(w.q), kv_cache=bits(w.kv), page_table=w.page_table.numpy(),
                                 seq_lens=w.seq_lens.numpy(), num_q_heads=w.num_q_heads,
                                 page_size=w.page_size, scale=w.scale, pt_cols=w.pt_cols)
    refs = [ref(wa), ref(wb)]
    g = _capture(lambda: m.run(out, lse))
    for rep in range(4):
        w = (wa, wb)[rep % 2]
        m.q.copy_(w.q)
        m.seq_lens.copy_(w.seq_lens)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o = out.float().cpu().numpy()
        l = lse.cpu().numpy()
        ro, rl = refs[rep % 2]
        assert np.all(np.isfinite(o))
        assert np.max(np.abs(o - ro)) <= 1.5e-2 and np.max(np.abs(l - rl)) <= 1e-3, "mla replay %d" % rep


def test_graph_replay_append():
    import oracle
    w = H.random_workload(77, kv_dtype="fp8_e4m3", B=4, max_len=200)
    x = DeviceInputs(w)
    pa = PagedAttention(w)
    T, Hkv, D = w.total_q, w.num_kv_heads, w.head_dim
    k_new = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    a = B.make_append_args(k_new=k_new, v_new=v_new, cu_new=x.cu_q_lens, seq_lens=x.seq_lens,
                           page_table=x.page_table, k_pool=x.k_pool, v_pool=x.v_pool,
                           k_descale=x.k_descale, v_descale=x.v_descale)
    g = _capture(lambda: B.pa_run_append(pa.plan, a, B.current_stream()))
    kp, vp = w.k_pool.numpy().copy(), w.v_pool.numpy().copy()
    for rep in range(3):
        kn = synth.normal_bf16(T * Hkv * D, 90 + rep, 1, 1).view(T, Hkv, D)
        vn = synth.normal_bf16(T * Hkv * D, 90 + rep, 2, 1).view(T, Hkv, D)
        k_new.copy_(kn)
        v_new.copy_(vn)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kp, vp = oracle.append(k_new=kn.view(torch.int16).numpy().view(np.uint16),
                               v_new=vn.view(torch.int16).numpy().view(np.uint16), k_pool=kp, v_pool=vp,
                               page_table=w.page_table.numpy(), cu_new=w.cu_q_lens.numpy(),
                               seq_lens=w.seq_lens.numpy(), num_kv_heads=Hkv, head_dim=D,
                               page_size=w.page_size, kv_dtype=oracle.KV_FP8_E4M3,
                               k_descale=w.k_descale, v_descale=w.v_descale, pt_cols=w.pt_cols)
        assert np.array_equal(x.k_pool.cpu().numpy(), kp) and np.array_equal(x.v_pool.cpu().numpy(), vp), \
            "append replay %d" % rep
