"""GPU parity of the head-split MLA decode (head groups of 33-64 heads: wave
pairs that split each 32-key tile's keys for the scores and the value
columns for the output) against the fp64 oracle:

- every page size at 33, 48, 64, 100 and 128 heads (partial head groups,
  pairs with no live head), lengths around the tile size (1, 31, 32, 33, 95)
  and longer ones, on the split and balanced schedules;
- rows whose running maximum moves far (the RoPE columns of the cache scaled
  up along the sequence, or only on the first key), so that the lazy rescale
  of the accumulator runs in both waves of a pair.  These rows are held to
  the bf16 rounding bound per element: with u = 2^-8, rounding P and O to
  bf16 moves an output by at most u (A + |O|), where A = sum_j p_j |v_j| is
  computed here in fp64 from the oracle's log-sum-exp; 1e-3 covers the fp32
  score, exp2 and accumulation error."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import MlaDecode
from tests.test_gpu_mla import LSE_TOL, ref, run_check

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -8
LENGTHS = [1, 31, 32, 33, 95, 257, 700]


@pytest.mark.parametrize("page", [16, 32, 64, 128])
@pytest.mark.parametrize("hq", [33, 48, 64, 100, 128])
def test_head_split_every_page_size(hq, page):
    w = synth.build_mla(name="mla_hs_%d_%d" % (hq, page), seq_lens=LENGTHS, num_q_heads=hq, page_size=page,
                        seed=1500 + hq + page, threads=2)
    r = ref(w)
    for s in (0, 2):
        run_check(w, num_splits=s, r=r)
    for cus in (0, 5):
        run_check(w, num_splits=-1, num_cus=cus, r=r)


def scale_rope(w, factor):
    """Multiply the 64 RoPE columns of key j of every sequence by factor(j, L)
    (scores move; the value columns stay as they are)."""
    pt = w.page_table.numpy()
    for b, n in enumerate(w.seq_lens.numpy()):
        n = int(n)
        j = np.arange(n)
        pages = torch.from_numpy(pt[b, j // w.page_size].astype(np.int64))
        slots = torch.from_numpy((j % w.page_size).astype(np.int64))
        f = torch.tensor([factor(int(x), n) for x in j], dtype=torch.float32)
        rows = w.kv[pages, slots].float()
        rows[:, 512:] *= f[:, None]
        w.kv[pages, slots] = rows.to(torch.bfloat16)


def weighted_abs_values(w, lse):
    """A[b, h, :] = sum_j p_j |v_j| with p_j = exp(scale q.k_j - LSE[b, h])."""
    q = w.q.double().numpy()
    kv = w.kv.double().numpy()
    pt = w.page_table.numpy()
    out = np.zeros((w.num_seqs, w.num_q_heads, 512))
    for b, n in enumerate(w.seq_lens.numpy()):
        n = int(n)
        if n == 0:
            continue
        j = np.arange(n)
        rows = kv[pt[b, j // w.page_size], j % w.page_size]
        p = np.exp(w.scale * (q[b] @ rows.T) - lse[b][:, None])
        out[b] = p @ np.abs(rows[:, :512])
    return out


@pytest.mark.parametrize("hq", [64, 128])
@pytest.mark.parametrize("shape", ["growing", "dominant_first"])
def test_head_split_moving_maximum(hq, shape):
    L = [700, 1300, 257, 64, 33]
    w = synth.build_mla(name="mla_hs_move", seq_lens=L, num_q_heads=hq, page_size=32, seed=1600 + hq,
                        threads=2)
    if shape == "growing":
        scale_rope(w, lambda j, n: 1.0 + 30.0 * j / max(n - 1, 1))
    else:
        scale_rope(w, lambda j, n: 30.0 if j == 0 else 1.0)
    ro, rl = ref(w)
    ro = ro.reshape(w.num_seqs, hq, 512)
    rl = rl.reshape(w.num_seqs, hq)
    bound = U_BF16 * (weighted_abs_values(w, rl) + np.abs(ro)) + 1e-3
    for s, cus in ((0, 0), (2, 0), (-1, 0), (-1, 3)):
        m = MlaDecode(w, num_splits=s, num_cus=cus)
        print("case", w.name, shape, "Hq", hq, "splits", m.num_splits, "cus", cus, flush=True)
        out, lse = m.run()
        torch.cuda.synchronize()
        o = out.float().cpu().numpy().astype(np.float64).reshape(ro.shape)
        l = lse.cpu().numpy().astype(np.float64).reshape(rl.shape)
        assert np.all(np.isfinite(o))
        excess = np.abs(o - ro) - bound
        i = int(np.argmax(excess))
        assert excess.flat[i] <= 0, "S%d: |dO| %.3g > %.3g (O %.4g)" % (
            m.num_splits, abs(o.flat[i] - ro.flat[i]), bound.flat[i], ro.flat[i])
        assert float(np.max(np.abs(l - rl))) <= LSE_TOL
