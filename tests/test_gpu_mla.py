"""GPU parity of MLA decode (pa_run_mla_decode) against the fp64 oracle:
random batches element by element over head counts 1..128 (one and two row
tiles per workgroup, one and two head groups), every page size, empty and
one-key sequences, forced and heuristic splits, softcap; the full-size MLA
workloads on sampled rows.  Tolerances as for bf16 attention."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import MlaDecode

pytestmark = pytest.mark.gpu

O_TOL = 1.5e-2
LSE_TOL = 1e-3


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def ref(w, rows=None):
    return oracle.mla_decode(q_bits=bits(w.q), kv_cache=bits(w.kv), page_table=w.page_table.numpy(),
                             seq_lens=w.seq_lens.numpy(), num_q_heads=w.num_q_heads,
                             page_size=w.page_size, scale=w.scale, rows=rows, pt_cols=w.pt_cols,
                             softcap=w.softcap)


def run_check(w, num_splits=0, num_cus=0, rows=None, r=None):
    m = MlaDecode(w, num_splits=num_splits, num_cus=num_cus)
    print("case", w.name, "Hq", w.num_q_heads, "page", w.page_size, "splits", m.num_splits, flush=True)
    out, lse = m.run()
    torch.cuda.synchronize()
    ro, rl = r if r is not None else ref(w, rows)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o.reshape(-1, 512)[rows]
        l = l.reshape(-1)[rows]
    ro = ro.reshape(o.shape)
    rl = rl.reshape(l.shape)
    assert np.all(np.isfinite(o)), "non-finite output"
    eo = float(np.max(np.abs(o - ro))) if o.size else 0.0
    both = np.isneginf(l) & np.isneginf(rl)
    el = float(np.max(np.where(both, 0.0, np.abs(l - rl)))) if l.size else 0.0
    assert eo <= O_TOL and el <= LSE_TOL, "%s S%d: max|dO| %.3g max|dLSE| %.3g" % (
        w.name, m.num_splits, eo, el)


@pytest.mark.parametrize("seed", range(12))
def test_mla_random(seed):
    rng = np.random.default_rng(1100 + seed)
    Hq = int(rng.choice([1, 8, 16, 32, 40, 64, 100, 128]))
    page = int(rng.choice([16, 32, 64, 128]))
    B = int(rng.integers(1, 6))
    L = rng.integers(0, 700, size=B)
    L[rng.random(B) < 0.2] = 1
    w = synth.build_mla(name="mla_rand%d" % seed, seq_lens=L, num_q_heads=Hq, page_size=page,
                        seed=1200 + seed, threads=1)
    if seed % 4 == 1:
        w.softcap = 1.5
    r = ref(w)
    for s in (0, 1, 3):
        run_check(w, num_splits=s, r=r)
    # balanced schedule on the device's grid and on tiny grids (items cut
    # into many pieces across workgroups)
    for cus in (0, 1, 3, 7):
        run_check(w, num_splits=-1, num_cus=cus, r=r)


def test_mla_long_sequence_many_splits():
    w = synth.build_mla(name="mla_long", seq_lens=[9000, 33], num_q_heads=64, page_size=64,
                        seed=1300, threads=4)
    r = ref(w)
    run_check(w, r=r)
    run_check(w, num_splits=7, r=r)
    run_check(w, num_splits=-1, r=r)
    run_check(w, num_splits=-1, num_cus=5, r=r)


@pytest.mark.slow
@pytest.mark.parametrize("make", [synth.mla_decode_h16, synth.mla_decode_h128])
def test_mla_full_size(make):
    w = make()
    rng = np.random.default_rng(5)
    rows = sorted(set(int(b) * w.num_q_heads + int(h) for b, h in
                      zip(rng.integers(0, w.num_seqs, 96), rng.integers(0, w.num_q_heads, 96))))
    run_check(w, rows=rows)
    run_check(w, rows=rows, num_splits=-1)
