"""Pins for the fp64 oracle: each checks it against something other than itself.

  * library routines: torch's CPU flash-attention operator in float64 (O and
    LSE), torch's float8_e4m3fn and bfloat16 casts;
  * closed forms: scale 0 gives prefix means and ln(count); one key gives V_0
    and s_0; identical keys give mean(V) and s + ln n;
  * invariants: physical-page permutation, split/merge over arbitrary key
    windows, GQA == MHA with replicated KV heads, decode row == last row of a
    full causal prefill, linearity in V, causal == non-causal at q_len 1,
    poisoned (NaN) slots outside the definition never read.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_attention_amd import synth
from tests import helpers as H

TOL = 1e-12


# --------------------------------------------------------------------------
# element formats
# --------------------------------------------------------------------------

def test_fp8_e4m3_all_codes_match_torch_cast():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = oracle.fp8_e4m3_to_double(c)
        want = float(ref[c])
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want, (c, got, want)


def test_fp8_e4m3_closed_form_landmarks():
    # OCP E4M3: bias 7, subnormal step 2^-9, max 448, S.1111.111 NaN, no inf
    assert oracle.fp8_e4m3_to_double(0x00) == 0.0
    assert oracle.fp8_e4m3_to_double(0x01) == 2.0 ** -9
    assert oracle.fp8_e4m3_to_double(0x07) == 7 * 2.0 ** -9
    assert oracle.fp8_e4m3_to_double(0x08) == 2.0 ** -6
    assert oracle.fp8_e4m3_to_double(0x38) == 1.0
    assert oracle.fp8_e4m3_to_double(0x7E) == 448.0
    assert oracle.fp8_e4m3_to_double(0xFE) == -448.0
    assert oracle.fp8_e4m3_to_double(0x78) == 256.0
    assert math.isnan(oracle.fp8_e4m3_to_double(0x7F))
    assert math.isnan(oracle.fp8_e4m3_to_double(0xFF))
    assert oracle.fp8_e4m3_to_double(0x80) == 0.0 and math.copysign(
        1, oracle.fp8_e4m3_to_double(0x80)) < 0


def test_bf16_decode_matches_torch_cast():
    rng = np.random.default_rng(0)
    codes = np.concatenate([rng.integers(0, 1 << 16, 4000), [0, 0x8000, 0x3F80, 0x7F7F,
                                                               0x0001, 0x807F]])
    ref = torch.from_numpy(codes.astype(np.int32).astype(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()
    for c, want in zip(codes, ref):
        got = oracle.bf16_to_double(int(c))
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want


# --------------------------------------------------------------------------
# P1: agreement with a library attention routine on gathered contiguous K/V
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_matches_library_attention_random(seed):
    kv = "fp8_e4m3" if seed % 4 == 3 else "bf16"
    w = H.random_workload(seed, kv_dtype=kv, causal=(seed % 3 != 2))
    o, lse = H.run_oracle(w)
    ro, rl = H.library_attention(w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o - ro)) < 1e-11
    assert np.max(np.abs(lse - rl)) < 1e-11


def test_matches_library_attention_tiny_mixed():
    w = synth.tiny_mixed()
    o, lse = H.run_oracle(w)
    ro, rl = H.library_attention(w)
    assert np.max(np.abs(o - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


# --------------------------------------------------------------------------
# P2-P4: closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_scale_zero_gives_prefix_means(seed):
    # scale 0: every visible key weighs the same, so O is the mean of V over the
    # visible set and LSE = ln |visible|.  Pins the causal offset, the tail
    # length and the head map (V differs per KV head).
    w = H.random_workload(seed, causal=(seed % 2 == 0), kv_dtype="bf16" if seed < 4 else "fp8_e4m3")
    o, lse = H.run_oracle(w, scale=0.0)
    kpool, vpool = H.decoded_pools(w)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_q_lens.numpy()
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        ql = int(cu[b + 1] - cu[b])
        _, v = H.contiguous_kv(w, b, kpool, vpool)
        csum = np.cumsum(v.numpy(), axis=0)   # [L, Hkv, D]
        for i in range(ql):
            t = int(cu[b]) + i
            n = (L - ql + i + 1) if w.causal else L
            for h in range(w.num_q_heads):
                want = csum[n - 1, h // G] / n
                assert np.max(np.abs(o[t, h] - want)) < TOL
                assert abs(lse[t, h] - math.log(n)) < TOL


def test_single_key_returns_v0_and_score():
    w = H.random_workload(3, B=3, decode=True, max_len=1)   # every L = 1
    o, lse = H.run_oracle(w)
    kpool, vpool = H.decoded_pools(w)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        k, v = H.contiguous_kv(w, b, kpool, vpool)
        for h in range(w.num_q_heads):
            q = w.q[b, h].to(torch.float64)
            s0 = w.scale * float(q @ k[0, h // G])
            assert np.max(np.abs(o[b, h] - v[0, h // G].numpy())) < TOL
            assert abs(lse[b, h] - s0) < 1e-12 * max(1.0, abs(s0))


def test_first_row_of_causal_prefill_sees_one_key():
    w = synth.tiny_mixed()
    o, lse = H.run_oracle(w)
    k, v = H.contiguous_kv(w, 0)
    for h in range(w.num_q_heads):
        s0 = w.scale * float(w.q[0, h].to(torch.float64) @ k[0, h // 2])
        assert np.max(np.abs(o[0, h] - v[0, h // 2].numpy())) < TOL
        assert abs(lse[0, h] - s0) < 1e-13


def test_identical_keys_give_mean_v_and_shifted_lse():
    w = H.random_workload(7, B=2, decode=True, max_len=60, G=2, Hkv=2, D=64)
    # overwrite every K row with the K row of (page_table[b,0], slot 0) of its head
    k = w.k_pool.clone()
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        first = k[int(w.page_table[b, 0]), 0].clone()
        for j in range(L):
            k[int(w.page_table[b, j // w.page_size]), j % w.page_size] = first
    w.k_pool = k
    o, lse = H.run_oracle(w)
    kpool, vpool = H.decoded_pools(w)
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        kk, vv = H.contiguous_kv(w, b, kpool, vpool)
        for h in range(w.num_q_heads):
            s = w.scale * float(w.q[b, h].to(torch.float64) @ kk[0, h // 2])
            assert np.max(np.abs(o[b, h] - vv[:, h // 2].mean(0).numpy())) < TOL
            assert abs(lse[b, h] - (s + math.log(L))) < 1e-12 * max(1, abs(s))


# --------------------------------------------------------------------------
# P5-P11: invariants
# --------------------------------------------------------------------------

def test_physical_page_permutation_is_bitwise_invariant():
    w = H.random_workload(11, B=4, max_len=200, page=16)
    o1, l1 = H.run_oracle(w)
    P = w.num_pages
    perm = torch.from_numpy(np.random.default_rng(5).permutation(P))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    # new pool row perm-index r holds old page perm[r]; old page p moves to inv[p]
    w.k_pool = w.k_pool[perm].contiguous()
    w.v_pool = w.v_pool[perm].contiguous()
    w.page_table = inv[w.page_table.to(torch.int64)].to(torch.int32)
    o2, l2 = H.run_oracle(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(4))
def test_split_merge_equals_unsplit(seed):
    w = H.random_workload(20 + seed, max_len=150, kv_dtype="bf16" if seed % 2 else "fp8_e4m3")
    o, lse = H.run_oracle(w)
    rng = np.random.default_rng(seed)
    Lmax = w.max_seq_len
    cuts = sorted(set([0, Lmax + 7] + list(rng.integers(0, Lmax + 1, size=4))))
    parts_o, parts_l = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        po, pl = H.run_oracle(w, key_begin=lo, key_end=hi)
        parts_o.append(po.reshape(-1, w.head_dim))
        parts_l.append(pl.reshape(-1))
    # an extra window beyond every sequence: empty for all rows (-inf)
    po, pl = H.run_oracle(w, key_begin=Lmax + 7, key_end=Lmax + 9)
    assert np.all(pl == -np.inf) and np.all(po == 0)
    parts_o.append(po.reshape(-1, w.head_dim))
    parts_l.append(pl.reshape(-1))
    mo, ml = oracle.merge(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(mo - o.reshape(-1, w.head_dim))) < TOL
    assert np.max(np.abs(ml - lse.reshape(-1))) < TOL


def test_gqa_equals_mha_with_replicated_kv_heads():
    w = H.random_workload(31, B=3, G=4, Hkv=2, D=64, page=16, max_len=70)
    o, lse = H.run_oracle(w)
    G = 4
    w.k_pool = w.k_pool.repeat_interleave(G, dim=2).contiguous()
    w.v_pool = w.v_pool.repeat_interleave(G, dim=2).contiguous()
    w.num_kv_heads = w.num_q_heads
    o2, l2 = H.run_oracle(w)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_decode_row_equals_last_row_of_full_prefill():
    # same keys: a causal prefill of L tokens and a decode of the last one
    L = [45, 90, 17]
    full = synth.build(name="full", seq_lens=L, q_lens=L, num_q_heads=4, num_kv_heads=2,
                       head_dim=64, page_size=16, seed=77, threads=1)
    of, lf = H.run_oracle(full)
    dec = synth.build(name="dec", seq_lens=L, q_lens=[1, 1, 1], num_q_heads=4, num_kv_heads=2,
                      head_dim=64, page_size=16, seed=77, threads=1)
    cu = full.cu_q_lens.numpy()
    q = torch.stack([full.q[cu[b + 1] - 1] for b in range(3)])
    dec.q = q
    dec.k_pool, dec.v_pool, dec.page_table = full.k_pool, full.v_pool, full.page_table
    od, ld = H.run_oracle(dec)
    for b in range(3):
        assert np.array_equal(od[b], of[cu[b + 1] - 1])
        assert np.array_equal(ld[b], lf[cu[b + 1] - 1])
    # a chunk of the last 10 tokens on 35 cached: rows equal the prefill tail
    ch = synth.build(name="chunk", seq_lens=L, q_lens=[10, 10, 10], num_q_heads=4,
                     num_kv_heads=2, head_dim=64, page_size=16, seed=77, threads=1)
    ch.q = torch.cat([full.q[cu[b + 1] - 10:cu[b + 1]] for b in range(3)])
    ch.k_pool, ch.v_pool, ch.page_table = full.k_pool, full.v_pool, full.page_table
    oc, lc = H.run_oracle(ch)
    for b in range(3):
        assert np.array_equal(oc[10 * b:10 * b + 10], of[cu[b + 1] - 10:cu[b + 1]])


def test_linear_in_v():
    w = H.random_workload(41, B=3, D=64, G=2, Hkv=2, page=16, max_len=50, poison=False)
    rng = np.random.default_rng(1)
    # V values k/8 with |k| <= 32: 2V + 1 stays exact in bf16
    vals = torch.from_numpy(rng.integers(-32, 33, size=w.v_pool.shape) / 8.0).to(torch.bfloat16)
    w.v_pool = vals
    o1, l1 = H.run_oracle(w)
    w.v_pool = (vals.to(torch.float64) * 2 + 1).to(torch.bfloat16)
    assert torch.equal(w.v_pool.to(torch.float64), vals.to(torch.float64) * 2 + 1)
    o2, l2 = H.run_oracle(w)
    assert np.max(np.abs(o2 - (2 * o1 + 1))) < 1e-12
    assert np.array_equal(l1, l2)


def test_causal_equals_noncausal_for_single_token_queries():
    w = H.random_workload(51, decode=True, max_len=300)
    o1, l1 = H.run_oracle(w, causal=True)
    o2, l2 = H.run_oracle(w, causal=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_poisoned_slots_are_never_read():
    w = H.random_workload(61, B=4, max_len=100, page=32)
    o1, l1 = H.run_oracle(w)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    w2 = H.random_workload(61, B=4, max_len=100, page=32, poison=False)
    o2, l2 = H.run_oracle(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_selection_matches_full_evaluation():
    w = synth.tiny_mixed()
    o, lse = H.run_oracle(w)
    rows = [0, 5, 37 * 4 - 1, 37 * 4, 37 * 4 + 3]
    ro, rl = H.run_oracle(w, rows=rows)
    for n, r in enumerate(rows):
        assert np.array_equal(ro[n], o.reshape(-1, w.head_dim)[r])
        assert rl[n] == lse.reshape(-1)[r]


def test_contract_violations_are_rejected():
    w = synth.tiny_mixed()
    bad = synth.tiny_mixed()
    bad.seq_lens = torch.tensor([36, 50], dtype=torch.int32)     # q_len 37 > L 36
    with pytest.raises(oracle.OracleError):
        H.run_oracle(bad)
    bad = synth.tiny_mixed()
    pt = bad.page_table.clone()
    pt[1, 0] = 16                                                  # outside the 16-page pool
    bad.page_table = pt
    with pytest.raises(oracle.OracleError):
        H.run_oracle(bad)
    bad = synth.tiny_mixed()
    bad.seq_lens = torch.tensor([37, 65], dtype=torch.int32)     # more than C * page keys
    with pytest.raises(oracle.OracleError):
        H.run_oracle(bad)
    # unused page-table columns may hold anything
    ok = synth.tiny_mixed()
    pt = ok.page_table.clone()
    pt[0, 3] = -12345
    ok.page_table = pt
    o1, _ = H.run_oracle(ok)
    o0, _ = H.run_oracle(w)
    assert np.array_equal(o0, o1)
