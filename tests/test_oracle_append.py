"""Pins of the oracle's KV-cache append and its E4M3 encoder (CPU only).

The encoder is checked against torch's float8_e4m3fn cast (an independent
round-to-nearest-even implementation) on every code, every midpoint between
neighbouring codes and points just beside them, and random values; the append
against a gather written here with numpy (bf16 rows restore a pool exactly,
fp8 rows land as torch-quantised codes, nothing else changes).  Planted
mistakes in a copy of the C source are each caught by these checks."""
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_attention_amd import synth
from tests import helpers as H

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")


def torch_e4m3(x: np.ndarray) -> np.ndarray:
    """torch's cast of binary32 values clamped to +-448."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encoder_probe_values() -> np.ndarray:
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = torch.tensor(finite, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2                        # exact ties (representable in binary32)
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(-np.inf))])
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.normal(0, 50, 4000), rng.uniform(-0.02, 0.02, 2000),
                           rng.uniform(400, 500, 200), [0.0, 448.0, 449.0, 464.0, 1e6]])
    x = np.concatenate([pos, mids, near, rand]).astype(np.float32)
    return np.concatenate([x, -x])


def encoder_failures() -> int:
    x = encoder_probe_values()
    want = torch_e4m3(x)
    got = np.array([oracle.fp8_e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    bad = int(np.sum(got != want))
    nan = np.float32(np.nan)
    for v in (nan, -nan):                                   # NaN keeps its sign, as torch's cast does
        bad += int(oracle.fp8_e4m3_encode(float(v)) != torch_e4m3(np.array([v]))[0])
    for c in range(256):                                   # decode-encode round trip
        if (c & 0x7F) != 0x7F and oracle.fp8_e4m3_encode(oracle.fp8_e4m3_to_double(c)) != c:
            bad += 1
    return bad


def positions(w):
    """(b, i, pos, page id, slot) of every new token: the last q_len tokens."""
    cu = w.cu_q_lens.numpy()
    L = w.seq_lens.numpy()
    pt = w.page_table.numpy()
    out = []
    for b in range(w.num_seqs):
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            pos = int(L[b]) - n + i
            out.append((b, int(cu[b]) + i, pos, int(pt[b, pos // w.page_size]), pos % w.page_size))
    return out


def append_failures(seeds=(3, 4, 6)) -> int:
    bad = 0
    for s in seeds:
        # bf16: the new rows are the pool's own rows at those positions; appending
        # them into a pool whose slots were poisoned must give the pool back
        w = H.random_workload(s, kv_dtype="bf16", max_len=120)
        k = w.k_pool.view(torch.int16).numpy().view(np.uint16)
        v = w.v_pool.view(torch.int16).numpy().view(np.uint16)
        pos = positions(w)
        T = int(w.cu_q_lens[-1])
        kn = np.zeros((T, w.num_kv_heads, w.head_dim), np.uint16)
        vn = np.zeros_like(kn)
        kp, vp = k.copy(), v.copy()
        for b, t, _, page, slot in pos:
            kn[t], vn[t] = k[page, slot], v[page, slot]
            kp[page, slot] = 0x7FC1
            vp[page, slot] = 0x7FC1
        ko, vo = oracle.append(k_new=kn, v_new=vn, k_pool=kp, v_pool=vp,
                               page_table=w.page_table.numpy(), cu_new=w.cu_q_lens.numpy(),
                               seq_lens=w.seq_lens.numpy(), num_kv_heads=w.num_kv_heads,
                               head_dim=w.head_dim, page_size=w.page_size, pt_cols=w.pt_cols)
        bad += int(np.sum(ko != k)) + int(np.sum(vo != v))
        # fp8: fresh rows land as torch-quantised codes; nothing else changes
        w8 = H.random_workload(s, kv_dtype="fp8_e4m3", max_len=120)
        k8 = w8.k_pool.numpy()
        v8 = w8.v_pool.numpy()
        T = int(w8.cu_q_lens[-1])
        shape = (T, w8.num_kv_heads, w8.head_dim)
        knb = synth.normal_bf16(int(np.prod(shape)), 50 + s, 1, 1).view(shape) * 3
        vnb = synth.normal_bf16(int(np.prod(shape)), 50 + s, 2, 1).view(shape) * 3
        ko, vo = oracle.append(k_new=knb.view(torch.int16).numpy().view(np.uint16),
                               v_new=vnb.view(torch.int16).numpy().view(np.uint16),
                               k_pool=k8, v_pool=v8, page_table=w8.page_table.numpy(),
                               cu_new=w8.cu_q_lens.numpy(), seq_lens=w8.seq_lens.numpy(),
                               num_kv_heads=w8.num_kv_heads, head_dim=w8.head_dim,
                               page_size=w8.page_size, kv_dtype=oracle.KV_FP8_E4M3,
                               k_descale=w8.k_descale, v_descale=w8.v_descale, pt_cols=w8.pt_cols)
        kq = torch_e4m3(knb.float().numpy() / np.float32(w8.k_descale))
        vq = torch_e4m3(vnb.float().numpy() / np.float32(w8.v_descale))
        ke, ve = k8.copy(), v8.copy()
        for b, t, _, page, slot in positions(w8):
            ke[page, slot], ve[page, slot] = kq[t], vq[t]
        bad += int(np.sum(ko != ke)) + int(np.sum(vo != ve))
    return bad


def test_encoder_matches_torch_and_round_trips():
    assert encoder_failures() == 0


def test_append_restores_bf16_and_quantises_fp8():
    assert append_failures() == 0


def test_append_rejects_contract_violations():
    w = H.random_workload(3, kv_dtype="bf16", max_len=50)
    T = int(w.cu_q_lens[-1])
    z = np.zeros((T, w.num_kv_heads, w.head_dim), np.uint16)
    short = w.seq_lens.numpy().copy()
    short[0] = int(w.cu_q_lens[1]) - 1                      # more new tokens than the length
    with pytest.raises(oracle.OracleError):
        oracle.append(k_new=z, v_new=z, k_pool=w.k_pool.view(torch.int16).numpy().view(np.uint16),
                      v_pool=w.v_pool.view(torch.int16).numpy().view(np.uint16),
                      page_table=w.page_table.numpy(), cu_new=w.cu_q_lens.numpy(), seq_lens=short,
                      num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                      pt_cols=w.pt_cols)


MUTANTS = {
    "position_off_by_one": ("const int64_t pos = L - n + i;", "const int64_t pos = L - n + i + 1 - (n == L);"),
    "first_token_as_base": ("const int64_t t = cu_new[b] + i;", "const int64_t t = cu_new[b] + (n - 1 - i);"),
    "head_slot_swapped": ("const int64_t dst = page * page_stride + (slot * H + g) * D + d;",
                          "const int64_t dst = page * page_stride + (g * pr->page_size + slot) * D + d;"),
    "descale_multiplied": ("const float kq = (float)pao_bf16_to_double(k_new[src]) / kd;",
                           "const float kq = (float)pao_bf16_to_double(k_new[src]) * kd;"),
    "ties_to_odd": ("(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    "ties_away": ("(err == best_err && (c & 1) == 0)", "(err == best_err)"),
    "sign_dropped": ("return (uint8_t)(best | (neg ? 0x80 : 0));", "return (uint8_t)best;"),
    "no_saturation": ("for (int c = 0; c < 0x7F; ++c) {", "for (int c = 0; c < 0x7E; ++c) {"),
    "nan_to_zero": ("if (isnan(x)) return", "if (0) return"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_append_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, "mutation anchor not unique: " + name
    src = tmp_path / "pa_oracle.c"
    src.write_text(text.replace(before, after))
    shutil.copy(os.path.join(os.path.dirname(SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    try:
        caught = encoder_failures() > 0 or append_failures() > 0
    except oracle.OracleError:
        caught = True
    assert caught, "planted mistake %s slipped through the append pins" % name
