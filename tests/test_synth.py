"""The seeded input generator: determinism and the structure the workloads state."""
import numpy as np
import torch

from paged_kv_gqa_attention_amd import synth


def test_same_seed_same_bytes_any_thread_count():
    a = synth.normal_bf16((1 << 22) * 3 + 17, seed=9, stream=2, threads=1)
    b = synth.normal_bf16((1 << 22) * 3 + 17, seed=9, stream=2, threads=8)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = synth.normal_bf16(1000, seed=10, stream=2)
    assert not torch.equal(a[:1000].view(torch.int16), c.view(torch.int16))


def test_tiny_mixed_layout():
    w = synth.tiny_mixed()
    assert w.page_table.shape == (2, 4) and w.num_pages == 16
    assert list(w.seq_lens) == [37, 50] and list(w.cu_q_lens) == [0, 37, 38]
    pt = w.page_table.numpy()
    live = list(pt[0, :3]) + list(pt[1, :4])
    assert len(set(live)) == 7 and pt[0, 3] == w.poison_page and w.poison_page not in live
    # NaN exactly in the dead slots
    k = w.k_pool.to(torch.float32)
    for b, L in enumerate([37, 50]):
        for j in range(64):
            page = pt[b, j // 16] if j // 16 < (L + 15) // 16 else None
            if page is None:
                continue
            row = k[page, j % 16]
            assert bool(torch.isnan(row).all()) == (j >= L)
    assert abs(w.scale - 0.125) < 1e-15


def test_named_workload_statistics_small_checks():
    # lengths within the stated ranges; all live pages distinct
    w = synth.decode_fp8_long(poison=False)
    L = w.seq_lens.numpy()
    assert L.min() >= 4096 and L.max() <= 32768 and w.is_decode
    assert w.k_pool.dtype == torch.uint8 and w.num_kv_heads == 2 and w.num_q_heads == 64
    pt = w.page_table.numpy()
    used = np.concatenate([pt[b, :(L[b] + 127) // 128] for b in range(64)])
    assert len(np.unique(used)) == used.size
    # descale = amax / 448 makes the largest code 448
    kv = w.k_pool.view(torch.float8_e4m3fn).to(torch.float32)
    assert float(kv.abs().max()) == 448.0


def test_mixed_order_and_shuffle():
    w = synth.mixed_24b(poison=False)
    ql = w.q_lens
    assert list(ql[:8]) == [1000] * 8 and np.all(ql[8:] == 1)
    L = w.seq_lens.numpy()
    assert np.all((L[:8] >= 1000) & (L[:8] <= 2000)) and np.all((L[8:] >= 1000) & (L[8:] <= 2000))
    s = synth.mixed_24b(shuffle=True, poison=False)
    assert sorted(s.q_lens.tolist()) == sorted(ql.tolist())
    assert s.q_lens.tolist() != ql.tolist()
