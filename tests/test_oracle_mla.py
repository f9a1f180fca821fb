"""Pins of the oracle's MLA decode (CPU only).

Against a dense evaluation written here with torch float64 library routines
(matmul, logsumexp, softmax) on the latent rows gathered through the page
table; against the pinned GQA oracle with one KV head whose K and V pools are
both the latent cache (head dim 576, first 512 outputs); a single-key closed
form.  Planted mistakes in a copy of the C source are each caught."""
import math
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_attention_amd import synth

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")
TOL = 1e-11
DK = synth.MLA_LATENT + synth.MLA_ROPE


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def run(w, rows=None, softcap=None):
    return oracle.mla_decode(q_bits=bits(w.q), kv_cache=bits(w.kv), page_table=w.page_table.numpy(),
                             seq_lens=w.seq_lens.numpy(), num_q_heads=w.num_q_heads,
                             page_size=w.page_size, scale=w.scale, rows=rows, pt_cols=w.pt_cols,
                             softcap=w.softcap if softcap is None else softcap)


def gathered(w, b):
    L = int(w.seq_lens[b])
    idx = [(int(w.page_table[b, j // w.page_size]), j % w.page_size) for j in range(L)]
    return torch.stack([w.kv[p, s] for p, s in idx]).to(torch.float64) if L else \
        torch.zeros(0, DK, dtype=torch.float64)


def dense(w):
    B, Hq = w.num_seqs, w.num_q_heads
    out = np.zeros((B, Hq, synth.MLA_LATENT))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        c = gathered(w, b)
        if c.shape[0] == 0:
            continue
        s = w.scale * (w.q[b].to(torch.float64) @ c.T)                 # [Hq, L]
        if w.softcap > 0:
            s = w.softcap * torch.tanh(s / w.softcap)
        lse[b] = torch.logsumexp(s, 1).numpy()
        out[b] = (torch.softmax(s, 1) @ c[:, :synth.MLA_LATENT]).numpy()
    return out, lse


def small(seed, Hq=16, page=16, lens=None):
    rng = np.random.default_rng(seed)
    L = lens if lens is not None else rng.integers(1, 90, size=int(rng.integers(1, 4)))
    return synth.build_mla(name="mla%d" % seed, seq_lens=L, num_q_heads=Hq, page_size=page,
                           seed=300 + seed, threads=1)


def failures() -> int:
    bad = 0
    for seed, Hq, page, cap in ((1, 16, 16, 0.0), (2, 8, 32, 0.0), (3, 32, 64, 0.0), (4, 16, 16, 1.5)):
        w = small(seed, Hq, page)
        w.scale = 0.06
        w.softcap = cap
        o, l = run(w)
        ro, rl = dense(w)
        bad += int(not (np.max(np.abs(o - ro)) < TOL and np.max(np.abs(l - rl)) < TOL))
    return bad


def test_matches_dense_library_evaluation():
    assert failures() == 0


def test_equals_gqa_oracle_with_latent_cache_as_k_and_v():
    w = small(5, Hq=8, page=16)
    o, l = run(w)
    kv = bits(w.kv).reshape(w.num_pages, w.page_size, 1, DK)
    B = w.num_seqs
    cu = np.arange(B + 1, dtype=np.int32)
    go, gl = oracle.attention(q_bits=bits(w.q).reshape(B, w.num_q_heads, DK), k_pool=kv, v_pool=kv,
                              page_table=w.page_table.numpy(), cu_q_lens=cu,
                              seq_lens=w.seq_lens.numpy(), num_q_heads=w.num_q_heads,
                              num_kv_heads=1, head_dim=DK, page_size=w.page_size, scale=w.scale,
                              causal=True, pt_cols=w.pt_cols)
    assert np.max(np.abs(o - go[..., :synth.MLA_LATENT])) < 1e-12
    assert np.max(np.abs(l - gl)) < 1e-12


def test_single_key_closed_form_and_empty_sequence():
    w = small(6, Hq=4, page=16, lens=[1, 0])
    o, l = run(w)
    c = gathered(w, 0)[0]
    for h in range(4):
        s = w.scale * float(w.q[0, h].to(torch.float64) @ c)
        assert abs(l[0, h] - s) < 1e-12 * max(1, abs(s))
        assert np.max(np.abs(o[0, h] - c[:synth.MLA_LATENT].numpy())) == 0
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def test_row_selection_and_rejections():
    w = small(7, Hq=8)
    o, l = run(w)
    rows = [0, 5, 7]
    so, sl = run(w, rows=rows)
    assert np.array_equal(so, o.reshape(-1, synth.MLA_LATENT)[rows])
    with pytest.raises(oracle.OracleError):
        run(w, rows=[w.num_seqs * 8])
    with pytest.raises(oracle.OracleError):
        run(w, softcap=-1.0)


MUTANTS = {
    "value_from_rope_side": ("o_row[d] += p * pao_bf16_to_double(c[d]);",
                             "o_row[d] += p * pao_bf16_to_double(c[d + pr->d_rope]);"),
    "rope_part_dropped": ("for (int64_t d = 0; d < Dk; ++d) dot +=", "for (int64_t d = 0; d < Dv; ++d) dot +="),
    "scale_dropped": ("s[j] = pr->scale * dot;", "s[j] = dot;"),
    "slot_shift": ("(j % pr->page_size) * Dk;\n    double dot", "((j + 1) % pr->page_size) * Dk;\n    double dot"),
    "page_stride_of_values": ("pr->kv_page_stride : (int64_t)pr->page_size * Dk;",
                              "pr->kv_page_stride : (int64_t)pr->page_size * Dv;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mla_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, "mutation anchor not unique: " + name
    src = tmp_path / "pa_oracle.c"
    src.write_text(text.replace(before, after))
    shutil.copy(os.path.join(os.path.dirname(SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    try:
        caught = failures() > 0
    except oracle.OracleError:
        caught = True
    assert caught, "planted mistake %s slipped through the MLA pins" % name
