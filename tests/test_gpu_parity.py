"""GPU parity: the HIP kernels of libpa.so against the fp64 oracle.

Every case compares element by element on the same seeded inputs:
max |O_gpu - O_oracle| <= 1.5e-2 (6e-2 with an fp8 cache) and
max |LSE_gpu - LSE_oracle| <= 1e-3, rows with no visible key excepted from
nothing (they must give O = 0 and LSE = -inf on both sides).
"""
import math

import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 1.5e-2, "fp8_e4m3": 6e-2}
LSE_TOL = 1e-3


def check(w, out, lse, ref_o, ref_l, rows=None, what=""):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o.reshape(-1, w.head_dim)[rows]
        l = l.reshape(-1)[rows]
    ref_o = ref_o.reshape(o.shape)
    ref_l = ref_l.reshape(l.shape)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    err_o = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    both_inf = np.isneginf(l) & np.isneginf(ref_l)
    dl = np.where(both_inf, 0.0, np.abs(l - ref_l))
    err_l = float(np.max(dl)) if dl.size else 0.0
    assert err_o <= O_TOL[w.kv_dtype], "%s: max|dO| = %.3g" % (what, err_o)
    assert err_l <= LSE_TOL, "%s: max|dLSE| = %.3g" % (what, err_l)
    return err_o, err_l


def run_and_check(w, mode, num_splits=0, rows=None, ref=None):
    print("case", w.name, mode, "splits", num_splits, flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=num_splits)
    out, lse = pa.run(mode, x)
    torch.cuda.synchronize()
    if ref is None:
        ref = H.run_oracle(w, rows=rows)
    return check(w, out, lse, ref[0], ref[1], rows=rows,
                 what="%s/%s/S%d" % (w.name, mode, pa.info.num_splits))


def test_tiny_mixed_all_schedules():
    w = synth.tiny_mixed()
    ref = H.run_oracle(w)
    run_and_check(w, "mixed", ref=ref)
    run_and_check(w, "prefill", ref=ref)
    run_and_check(w, "mixed", num_splits=2, ref=ref)


def test_tiny_decode_row_through_decode_entry():
    # the decode row of the tiny mixed batch (L = 50, q_len 1) on its own
    full = synth.tiny_mixed()
    w = synth.build(name="tiny_decode", seq_lens=[50], q_lens=[1], num_q_heads=4,
                    num_kv_heads=2, head_dim=64, page_size=16, seed=1, pt_cols=4,
                    num_pages=16, scale=1.0 / 8.0, threads=1)
    w.q = full.q[37:38].clone()
    w.k_pool, w.v_pool = full.k_pool, full.v_pool
    w.page_table = full.page_table[1:2].clone()
    ref = H.run_oracle(w)
    fo, fl = H.run_oracle(full)
    assert np.array_equal(ref[0][0], fo[37]) and np.array_equal(ref[1][0], fl[37])
    for s in (1, 2, 4):
        run_and_check(w, "decode", num_splits=s, ref=ref)
        run_and_check(w, "mixed", num_splits=s, ref=ref)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_and_mixed(seed):
    kv = "fp8_e4m3" if seed % 3 == 2 else "bf16"
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    w = H.random_workload(seed, kv_dtype=kv, causal=(seed % 4 != 3), max_len=300, G=G,
                          Hkv=int(rng.choice([1, 2])))
    ref = H.run_oracle(w)
    run_and_check(w, "prefill", ref=ref)
    run_and_check(w, "mixed", ref=ref)
    run_and_check(w, "mixed", num_splits=3, ref=ref)


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    kv = "fp8_e4m3" if seed % 2 else "bf16"
    rng = np.random.default_rng(100 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    w = H.random_workload(200 + seed, kv_dtype=kv, decode=True, max_len=900, G=G,
                          Hkv=int(rng.choice([1, 2, 3])), B=int(rng.integers(1, 9)))
    ref = H.run_oracle(w)
    for s in (0, 1, 2, 5):
        run_and_check(w, "decode", num_splits=s, ref=ref)
    run_and_check(w, "mixed", ref=ref)


@pytest.mark.parametrize("mode", ["decode", "mixed"])
def test_sequences_longer_than_the_planned_max(mode):
    # the plan's split windows cover max_seq_len = 1024; sequences run to
    # about 3,000 keys, so the last window takes every key past 768
    L = [3000, 1024, 1500, 7, 2049]
    w = synth.build(name="past_max_" + mode, seq_lens=L, q_lens=[1] * 5, num_q_heads=16,
                    num_kv_heads=4, head_dim=128, page_size=16, seed=61, threads=1)
    ref = H.run_oracle(w)
    for splits in (3, 4):
        pa = PagedAttention(w, num_splits=splits, max_seq_len=1024)
        print("case", w.name, "splits", pa.info.num_splits, "window", pa.info.split_keys, flush=True)
        assert (pa.info.num_splits - 1) * pa.info.split_keys < 1024   # the last window starts inside
        x = DeviceInputs(w)
        out, lse = pa.run(mode, x)
        torch.cuda.synchronize()
        check(w, out, lse, ref[0], ref[1], what="%s/S%d" % (w.name, splits))
