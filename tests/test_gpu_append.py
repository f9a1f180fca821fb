"""GPU parity of the KV-cache append (pa_run_append) against the oracle.

The pools after the append must equal the oracle's byte for byte (bf16 rows
are copied; fp8 codes are an integer decision both sides take from the same
binary32 quotient).  Attention over the appended pools is then checked against
the oracle to the usual tolerances, closing the append -> attend loop.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_attention_amd import binding as B
from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def np_bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def spread_bf16(n: int, seed: int, lo_exp: int = -14, hi_exp: int = 10) -> torch.Tensor:
    """bf16 values with random sign and mantissa over a wide exponent range, so
    that quotients by a descale land on E4M3 subnormals, normals, exact ties
    and beyond the saturation point."""
    rng = np.random.default_rng(seed)
    e = rng.integers(lo_exp + 127, hi_exp + 127, size=n).astype(np.uint16)
    m = rng.integers(0, 128, size=n).astype(np.uint16)
    s = rng.integers(0, 2, size=n).astype(np.uint16)
    return torch.from_numpy(((s << 15) | (e << 7) | m).view(np.int16)).view(torch.bfloat16)


def new_rows(w, seed: int, spread: bool, stride_pad: int = 0):
    T = w.total_q
    n = T * w.num_kv_heads * w.head_dim
    if spread:
        k = spread_bf16(n, seed)
        v = spread_bf16(n, seed + 1)
    else:
        # standard normal, as the workloads' K/V (the output tolerances assume it)
        k = synth.normal_bf16(n, seed, 1, 1)
        v = synth.normal_bf16(n, seed, 2, 1)
    k = k.view(T, w.num_kv_heads * w.head_dim)
    v = v.view(T, w.num_kv_heads * w.head_dim)
    if stride_pad:
        # rows inside a wider buffer (as from a fused QKV projection)
        pad = torch.full((T, stride_pad), float("nan"), dtype=torch.bfloat16)
        k = torch.cat([k, pad], 1)
        v = torch.cat([v, pad], 1)
    return k, v


def gpu_append(w, k_new, v_new, pools=None, max_total_q=None, seq_lens=None, cu_new=None):
    """Append on the GPU into device copies of w's pools; returns (x, k, v)."""
    print("append", w.name, w.kv_dtype, "D", w.head_dim, "Hkv", w.num_kv_heads,
          "page", w.page_size, "T", w.total_q, flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, max_total_q=max_total_q)
    kd = k_new.cuda()
    vd = v_new.cuda()
    stride = k_new.shape[1] if k_new.shape[1] != w.num_kv_heads * w.head_dim else 0
    a = B.make_append_args(k_new=kd, v_new=vd, new_stride_t=stride,
                           cu_new=x.cu_q_lens if cu_new is None else cu_new.cuda(),
                           seq_lens=x.seq_lens if seq_lens is None else seq_lens.cuda(),
                           page_table=x.page_table, k_pool=x.k_pool, v_pool=x.v_pool,
                           k_descale=x.k_descale, v_descale=x.v_descale)
    B.pa_run_append(pa.plan, a, B.current_stream())
    torch.cuda.synchronize()
    return x, pa


def oracle_append(w, k_new, v_new, cu_new=None, seq_lens=None):
    Hkv, D = w.num_kv_heads, w.head_dim
    kn = np_bits(k_new[:, :Hkv * D]).reshape(-1, Hkv, D)
    vn = np_bits(v_new[:, :Hkv * D]).reshape(-1, Hkv, D)
    return oracle.append(k_new=kn, v_new=vn, k_pool=np_bits(w.k_pool), v_pool=np_bits(w.v_pool),
                         page_table=w.page_table.numpy(),
                         cu_new=w.cu_q_lens.numpy() if cu_new is None else cu_new,
                         seq_lens=w.seq_lens.numpy() if seq_lens is None else seq_lens,
                         num_kv_heads=Hkv, head_dim=D, page_size=w.page_size,
                         kv_dtype=oracle.KV_BF16 if w.kv_dtype == "bf16" else oracle.KV_FP8_E4M3,
                         k_descale=w.k_descale, v_descale=w.v_descale, pt_cols=w.pt_cols)


def assert_pools_equal(x, ko, vo, what):
    kg, vg = np_bits(x.k_pool), np_bits(x.v_pool)
    nk = int(np.sum(kg != ko))
    nv = int(np.sum(vg != vo))
    detail = []
    for name, g, o in (("K", kg, ko), ("V", vg, vo)):
        idx = np.flatnonzero(g.reshape(-1) != o.reshape(-1))[:6]
        detail += ["%s[%d] gpu %#x oracle %#x" % (name, i, g.reshape(-1)[i], o.reshape(-1)[i])
                   for i in idx]
    assert nk == 0 and nv == 0, "%s: %d K and %d V elements differ; %s" % (
        what, nk, nv, "; ".join(detail))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_random_append_then_attend(seed, kv):
    w = H.random_workload(200 + seed, kv_dtype=kv, max_len=300)
    k_new, v_new = new_rows(w, seed, spread=False, stride_pad=8 * (seed % 3))
    x, pa = gpu_append(w, k_new, v_new)
    ko, vo = oracle_append(w, k_new, v_new)
    assert_pools_equal(x, ko, vo, "%s/%s" % (w.name, kv))
    # attention over the appended cache, GPU against oracle
    w2 = dataclasses.replace(w)
    if kv == "bf16":
        w2.k_pool = torch.from_numpy(ko.view(np.int16)).view(torch.bfloat16)
        w2.v_pool = torch.from_numpy(vo.view(np.int16)).view(torch.bfloat16)
    else:
        w2.k_pool = torch.from_numpy(ko)
        w2.v_pool = torch.from_numpy(vo)
    out, lse = pa.run("mixed", x)
    torch.cuda.synchronize()
    ref = H.run_oracle(w2)
    check(w2, out, lse, ref[0], ref[1], what="append+mixed %s/%s" % (w.name, kv))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_fp8_encoder_edge_values(D):
    # quotients across subnormals, ties, saturation, NaN and infinities
    w = H.random_workload(300 + D, kv_dtype="fp8_e4m3", D=D, max_len=200)
    w.k_descale = 0.125          # a power of two: K quotients hit exact ties often
    k_new, v_new = new_rows(w, D, spread=True)
    flat = k_new.view(-1)
    specials = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 448.0,
                             -464.0, 1e-30], dtype=torch.bfloat16)
    flat[:specials.numel()] = specials[:flat.numel()]
    x, _ = gpu_append(w, k_new, v_new)
    ko, vo = oracle_append(w, k_new, v_new)
    assert_pools_equal(x, ko, vo, "spread fp8 D=%d" % D)


def test_full_size_mixed_batch_append():
    for kv in ("bf16", "fp8_e4m3"):
        w = synth.mixed_24b(kv_dtype=kv)
        k_new, v_new = new_rows(w, 11, spread=False)
        x, _ = gpu_append(w, k_new, v_new)
        ko, vo = oracle_append(w, k_new, v_new)
        assert_pools_equal(x, ko, vo, "mixed_24b %s" % kv)


def test_contract_violations_and_row_cap_write_nothing():
    w = H.random_workload(400, kv_dtype="bf16", B=3, max_len=60, decode=False)
    ql = w.q_lens.astype(np.int64)
    L = w.seq_lens.numpy().astype(np.int64)
    k_new, v_new = new_rows(w, 5, spread=False)
    # sequence 0 claims more new tokens than its length: only its last L0 land
    bad_L = L.copy()
    bad_L[0] = max(0, int(ql[0]) - 2)
    # the plan's row cap stops before the last sequence's rows
    cap = int(w.cu_q_lens[-1]) - 1
    x, _ = gpu_append(w, k_new, v_new, seq_lens=torch.from_numpy(bad_L.astype(np.int32)),
                      max_total_q=max(cap, 1))
    keep = np.ones(w.total_q, dtype=bool)
    cu = w.cu_q_lens.numpy()
    keep[cu[0]:cu[0] + (int(ql[0]) - int(bad_L[0]))] = False      # negative positions
    keep[cap:] = False                                               # rows past the cap
    kept_ql = np.array([int(np.sum(keep[cu[b]:cu[b + 1]])) for b in range(w.num_seqs)])
    # the oracle's view of what must land: the kept rows, lengths shortened
    # by the rows dropped at the end of the last sequence
    exp_L = bad_L.copy()
    last = w.num_seqs - 1
    exp_L[last] -= int(np.sum(~keep[cu[last]:cu[last + 1]]))
    cu2 = np.concatenate([[0], np.cumsum(kept_ql)]).astype(np.int32)
    idx = torch.from_numpy(np.nonzero(keep)[0])
    ko, vo = oracle_append(w, k_new[idx], v_new[idx], cu_new=cu2, seq_lens=exp_L.astype(np.int32))
    assert_pools_equal(x, ko, vo, "contract violations")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_page_ids_outside_the_pool_are_not_written(kv):
    # sequence 1's last live page-table column names a page past the pool (or
    # -1): the new rows that land there are skipped, every other row lands
    w = H.random_workload(410 + (kv == "fp8_e4m3"), kv_dtype=kv, B=3, max_len=90, decode=False)
    ql = w.q_lens.astype(np.int64)
    L = w.seq_lens.numpy().astype(np.int64)
    k_new, v_new = new_rows(w, 7, spread=False)
    col = int((L[1] - 1) // w.page_size)
    for bad in (w.num_pages + 7, -1):
        print("append bad page id", bad, kv, flush=True)
        x = DeviceInputs(w)
        x.page_table[1, col] = bad
        pa = PagedAttention(w)
        a = B.make_append_args(k_new=k_new.cuda(), v_new=v_new.cuda(), cu_new=x.cu_q_lens,
                               seq_lens=x.seq_lens, page_table=x.page_table, k_pool=x.k_pool,
                               v_pool=x.v_pool, k_descale=x.k_descale, v_descale=x.v_descale)
        B.pa_run_append(pa.plan, a, B.current_stream())
        torch.cuda.synchronize()
        # expected: sequence 1 without its new rows on that page (they are its
        # last ones, so the others keep their positions)
        cu = w.cu_q_lens.numpy()
        pos = L[1] - ql[1] + np.arange(ql[1])
        drop = int(np.sum(pos // w.page_size == col))
        keep = np.ones(w.total_q, dtype=bool)
        keep[cu[2] - drop:cu[2]] = False
        exp_L = L.copy()
        exp_L[1] -= drop
        kept_ql = np.array([int(np.sum(keep[cu[b]:cu[b + 1]])) for b in range(w.num_seqs)])
        cu2 = np.concatenate([[0], np.cumsum(kept_ql)]).astype(np.int32)
        idx = torch.from_numpy(np.nonzero(keep)[0])
        ko, vo = oracle_append(w, k_new[idx], v_new[idx], cu_new=cu2, seq_lens=exp_L.astype(np.int32))
        assert drop > 0
        assert_pools_equal(x, ko, vo, "page id %d" % bad)


@pytest.mark.parametrize("descale", [1.0, 0.125, 0.0123, 3.7])
def test_fp8_encoder_every_bf16_value(descale):
    # every bf16 bit pattern (NaN payloads, infinities, subnormals, both zeros)
    # divided by a descale and encoded, against the oracle
    w = synth.build(name="every_bf16", seq_lens=[200, 100], q_lens=[150, 60], num_q_heads=4,
                    num_kv_heads=2, head_dim=256, page_size=16, seed=77, kv_dtype="fp8_e4m3",
                    threads=1)
    w.k_descale = descale
    w.v_descale = descale * 0.5
    n = w.total_q * w.num_kv_heads * w.head_dim
    assert n >= 1 << 16
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(5)
    kb = np.concatenate([allbits, rng.integers(0, 1 << 16, n - (1 << 16)).astype(np.uint16)])
    vb = rng.permutation(kb)
    k_new = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).view(w.total_q, -1)
    v_new = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).view(w.total_q, -1)
    x, _ = gpu_append(w, k_new, v_new)
    ko, vo = oracle_append(w, k_new, v_new)
    assert_pools_equal(x, ko, vo, "every bf16, descale %g" % descale)
