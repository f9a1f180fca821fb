"""Pins of the oracle's logit soft-capping (CPU only).

With a cap c > 0 every scaled score s = scale * q.k becomes c * tanh(s / c)
before the mask and the softmax.  Pinned against a brute-force evaluation
written here with torch/numpy library routines on gathered K/V, a closed form
(identical keys), the limit c -> infinity, and argument checks; planted
mistakes in a copy of the C source are each caught."""
import math
import os
import shutil

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from tests import helpers as H

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")
TOL = 1e-11


def brute_force(w, cap):
    """Dense per-sequence evaluation: S = scale Q K^T (float64 matmul), capped
    with np.tanh, masked bottom-right, softmax through scipy's logsumexp."""
    kpool, vpool = H.decoded_pools(w)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_q_lens.numpy()
    T, Hq, D = w.q.shape
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for b in range(w.num_seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        ql, L = hi - lo, int(w.seq_lens[b])
        if ql == 0:
            continue
        k, v = H.contiguous_kv(w, b, kpool, vpool)            # [L, Hkv, D]
        for h in range(Hq):
            q = w.q[lo:hi, h].to(torch.float64)                # [ql, D]
            s = (w.scale * (q @ k[:, h // G].T)).numpy()       # [ql, L]
            if cap > 0:
                s = cap * np.tanh(s / cap)
            if w.causal:
                i = np.arange(ql)[:, None]
                j = np.arange(L)[None, :]
                s = np.where(j <= L - ql + i, s, -np.inf)
            l = logsumexp(s, axis=1)
            p = np.exp(s - l[:, None])
            out[lo:hi, h] = p @ v[:, h // G].numpy()
            lse[lo:hi, h] = l
    return out, lse


def failures(cases=((3, "bf16", True, 5.0), (4, "fp8_e4m3", True, 30.0),
                    (5, "bf16", False, 2.0), (6, "bf16", True, 50.0))) -> int:
    bad = 0
    for seed, kv, causal, cap in cases:
        w = H.random_workload(600 + seed, kv_dtype=kv, causal=causal, max_len=70)
        w.scale = 0.5               # larger scores, so that the cap bends them
        w.softcap = cap
        o, l = H.run_oracle(w)
        ro, rl = brute_force(w, cap)
        bad += int(not (np.max(np.abs(o - ro)) < TOL and np.max(np.abs(l - rl)) < TOL))
    return bad


def identical_key_failures() -> int:
    w = H.random_workload(17, B=2, decode=True, max_len=60, G=2, Hkv=2, D=64)
    w.scale = 0.7
    cap = 3.0
    k = w.k_pool.clone()
    for b in range(w.num_seqs):
        first = k[int(w.page_table[b, 0]), 0].clone()
        for j in range(int(w.seq_lens[b])):
            k[int(w.page_table[b, j // w.page_size]), j % w.page_size] = first
    w.k_pool = k
    o, lse = H.run_oracle(w, softcap=cap)
    kpool, vpool = H.decoded_pools(w)
    bad = 0
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        kk, vv = H.contiguous_kv(w, b, kpool, vpool)
        for h in range(w.num_q_heads):
            s = w.scale * float(w.q[b, h].to(torch.float64) @ kk[0, h // 2])
            want = cap * math.tanh(s / cap) + math.log(L)
            bad += int(abs(lse[b, h] - want) > 1e-12 * max(1.0, abs(want)))
            bad += int(np.max(np.abs(o[b, h] - vv[:, h // 2].mean(0).numpy())) > TOL)
    return bad


def test_softcap_matches_brute_force():
    assert failures() == 0


def test_softcap_identical_keys_closed_form():
    assert identical_key_failures() == 0


def test_huge_cap_is_no_cap():
    w = H.random_workload(9, max_len=60)
    w.scale = 0.5
    o0, l0 = H.run_oracle(w, softcap=0.0)
    o1, l1 = H.run_oracle(w, softcap=1e9)
    assert np.max(np.abs(o0 - o1)) < 1e-9 and np.max(np.abs(l0 - l1)) < 1e-9


@pytest.mark.parametrize("cap", [-1.0, float("nan"), float("inf")])
def test_bad_cap_is_rejected(cap):
    w = H.random_workload(9, max_len=20)
    with pytest.raises(oracle.OracleError):
        H.run_oracle(w, softcap=cap)


MUTANTS = {
    "cap_on_unscaled_dot": ("pr->softcap * tanh(s[j - lo] / pr->softcap);",
                            "pr->softcap * tanh(dot / pr->softcap);"),
    "cap_factor_dropped": ("pr->softcap * tanh(s[j - lo] / pr->softcap);",
                           "tanh(s[j - lo] / pr->softcap);"),
    "cap_inverted": ("pr->softcap * tanh(s[j - lo] / pr->softcap);",
                     "pr->softcap * tanh(s[j - lo] * pr->softcap);"),
    "cap_ignored": ("if (pr->softcap > 0.0) s[j - lo]", "if (0) s[j - lo]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_softcap_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, "mutation anchor not unique: " + name
    src = tmp_path / "pa_oracle.c"
    src.write_text(text.replace(before, after))
    shutil.copy(os.path.join(os.path.dirname(SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    assert failures() > 0 or identical_key_failures() > 0, \
        "planted mistake %s slipped through the softcap pins" % name
