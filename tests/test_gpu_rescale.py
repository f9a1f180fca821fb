"""GPU parity where the running row maximum moves a lot, so that the lazy
rescale of the accumulator (taken only when the row maximum grows by more
than 8 in log2 units) and its per-lane threshold test run many times:

- keys whose magnitude grows along the sequence (the row maximum climbs by
  tens of log2 units from the first keys to the last);
- a dominant first key (every later probability underflows to zero);
- queries scaled far up (each row's probabilities peak on a single key).

Every schedule is covered: the streamed prefill (head dim 64, 128), the
row-split prefill (head dim 256), the row-split and key-split items of mixed
batches, split and balanced decode, and the ring decode of an fp8 cache at
head dim 256.  The oracle runs on the same scaled bf16 values.

The fixed 1.5e-2 bound of the other parity tests assumes that the bf16
rounding of the probabilities averages out over many keys; on these rows one
key can carry almost all the weight, so each element is held to the bound the
arithmetic gives instead.  With u = 2^-8, the unit roundoff of bf16 (8
significand bits), P rounded to bf16 moves sum_j p_j v_j / l by at most
u * sum_j p_j |v_j| / l, and rounding O to bf16 adds at most u * |O|:

    |O_gpu - O| <= u * (A + |O|) + 1e-3,   A = sum_j p_j |v_j| / l,

where A is the oracle's output on the same inputs with |V| in place of V, and
1e-3 covers the fp32 score, exp2 and accumulation error.  LSE keeps 1e-3."""
import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
LSE_TOL = 1e-3


def abs_values(w):
    """The workload with every V element replaced by its magnitude (sign bit
    cleared: bit 15 of a bf16, bit 7 of an E4M3 byte)."""
    if w.kv_dtype == "bf16":
        bits = w.v_pool.view(torch.int16) & 0x7FFF
        v = bits.view(torch.bfloat16)
    else:
        v = w.v_pool & 0x7F
    return dataclasses.replace(w, v_pool=v.clone())


def run_and_check(w, mode, num_splits=0, ref=None):
    """Run one schedule and check every element against the bound above.
    ref = (O, LSE, A) from the oracle, computed once per workload."""
    print("case", w.name, mode, "splits", num_splits, flush=True)
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=num_splits)
    out, lse = pa.run(mode, x)
    torch.cuda.synchronize()
    if ref is None:
        ref = oracle_refs(w)
    ref_o, ref_l, a = ref
    o = out.float().cpu().numpy().astype(np.float64).reshape(ref_o.shape)
    l = lse.float().cpu().numpy().astype(np.float64).reshape(ref_l.shape)
    what = "%s/%s/S%d" % (w.name, mode, pa.info.num_splits)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    bound = U_BF16 * (a + np.abs(ref_o)) + 1e-3
    excess = np.abs(o - ref_o) - bound
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, "%s: |dO| = %.3g > %.3g at %d (O = %.4g, A = %.4g)" % (
        what, abs(o.flat[i] - ref_o.flat[i]), bound.flat[i], i, ref_o.flat[i], a.flat[i])
    both_inf = np.isneginf(l) & np.isneginf(ref_l)
    dl = np.where(both_inf, 0.0, np.abs(l - ref_l))
    assert float(np.max(dl)) <= LSE_TOL, "%s: max|dLSE| = %.3g" % (what, float(np.max(dl)))
    return ref


def oracle_refs(w):
    ref_o, ref_l = H.run_oracle(w)
    a, _ = H.run_oracle(abs_values(w))
    return ref_o, ref_l, a


def scale_keys(w, factor):
    """Multiply key j of every sequence by factor(j, L) in the bf16 pool."""
    pt = w.page_table.numpy()
    lens = w.seq_lens.numpy()
    k = w.k_pool
    for b in range(w.num_seqs):
        n = int(lens[b])
        if n == 0:
            continue
        j = np.arange(n)
        pages = torch.from_numpy(pt[b, j // w.page_size].astype(np.int64))
        slots = torch.from_numpy((j % w.page_size).astype(np.int64))
        f = torch.tensor([factor(int(x), n) for x in j], dtype=torch.float32)
        rows = k[pages, slots].float() * f[:, None, None]
        k[pages, slots] = rows.to(torch.bfloat16)


def growing(j, n):
    return 1.0 + 12.0 * j / max(n - 1, 1)


def dominant_first(j, n):
    return 16.0 if j == 0 else 1.0


def build(hd, q_lens, seq_lens, seed, kv_dtype="bf16", G=4):
    return synth.build(name="rescale_d%d" % hd, seq_lens=seq_lens, q_lens=q_lens,
                       num_q_heads=2 * G, num_kv_heads=2, head_dim=hd, page_size=32,
                       seed=seed, kv_dtype=kv_dtype)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("shape", ["growing", "dominant_first"])
def test_prefill_and_mixed_with_moving_maximum(hd, shape):
    L = [700, 1300, 257, 64]
    w = build(hd, L, L, seed=hd + (0 if shape == "growing" else 1))
    scale_keys(w, growing if shape == "growing" else dominant_first)
    ref = run_and_check(w, "prefill")
    run_and_check(w, "mixed", ref=ref)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("shape", ["growing", "dominant_first"])
def test_decode_with_moving_maximum(hd, shape):
    rng = np.random.default_rng(hd)
    L = rng.integers(200, 3000, size=12)
    w = build(hd, [1] * 12, L, seed=10 + hd + (0 if shape == "growing" else 1))
    scale_keys(w, growing if shape == "growing" else dominant_first)
    ref = run_and_check(w, "decode")
    run_and_check(w, "decode", num_splits=3, ref=ref)
    run_and_check(w, "decode", num_splits=-1, ref=ref)
    # a chunk and decode rows in one mixed batch (both item kinds)
    wm = build(hd, [1] * 11 + [150], L, seed=30 + hd)
    scale_keys(wm, growing if shape == "growing" else dominant_first)
    run_and_check(wm, "mixed")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("hd", [128, 256])
def test_peaked_queries(kv, hd):
    # queries scaled up 8x: scaled scores with a spread of tens of log2 units
    rng = np.random.default_rng(7 + hd)
    L = rng.integers(100, 2500, size=8)
    G = 32 if hd == 256 else 4
    w = build(hd, [1] * 8, L, seed=50 + hd, kv_dtype=kv, G=G)
    w.q = (w.q.float() * 8.0).to(torch.bfloat16)
    ref = run_and_check(w, "decode")
    run_and_check(w, "decode", num_splits=-1, ref=ref)
    Lp = [int(x) for x in L[:4] // 2]
    wp = build(hd, Lp, Lp, seed=60 + hd, kv_dtype=kv)
    wp.q = (wp.q.float() * 8.0).to(torch.bfloat16)
    run_and_check(wp, "prefill")
