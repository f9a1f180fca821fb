"""Shared test helpers: workload marshalling and independent reference checks.

Nothing here is imported by the product package or by the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from paged_kv_gqa_attention_amd import synth


def bits(w: synth.Workload):
    """numpy views of a workload: q bf16 bits, K/V pools (bf16 bits or fp8 bytes)."""
    return oracle.workload_arrays(w)


def run_oracle(w: synth.Workload, rows=None, key_begin=0, key_end=-1, causal=None,
               scale=None, threads=0, softcap=None):
    return oracle.attention_workload(w, rows=rows, key_begin=key_begin, key_end=key_end,
                                     causal=causal, scale=scale, threads=threads,
                                     softcap=softcap)


def cover_rows(w: synth.Workload, q_block_tokens: int, seed: int = 5):
    """Flat (t*Hq + h) rows that touch every work item of a launch: for each
    sequence, each q-block of q_block_tokens query tokens and each slice of
    32 // G tokens inside it (the packed rows one wave owns), one random token
    with one random query head of every KV head; plus each sequence's first
    and last query token at every head.  Sequences with q_len * G <= 32 (one
    wave's rows) contribute all their rows."""
    rng = np.random.default_rng(seed)
    cu = w.cu_q_lens.numpy()
    Hq, Hkv = w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    per_wave = max(1, 32 // G)
    rows = set()
    for b in range(w.num_seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        if (hi - lo) * G <= 32:
            rows.update(t * Hq + h for t in range(lo, hi) for h in range(Hq))
            continue
        for t in (lo, hi - 1):
            rows.update(t * Hq + h for h in range(Hq))
        for q0 in range(lo, hi, q_block_tokens):
            q1 = min(hi, q0 + q_block_tokens)
            for s0 in range(q0, q1, per_wave):
                t = int(rng.integers(s0, min(q1, s0 + per_wave)))
                for g in range(Hkv):
                    rows.add(t * Hq + g * G + int(rng.integers(0, G)))
    return sorted(rows)


def decoded_pools(w: synth.Workload):
    """K/V pools as float64 tensors, decoded with torch's own dtype casts."""
    if w.kv_dtype == "bf16":
        return w.k_pool.to(torch.float64), w.v_pool.to(torch.float64)
    k = w.k_pool.view(torch.float8_e4m3fn).to(torch.float64) * w.k_descale
    v = w.v_pool.view(torch.float8_e4m3fn).to(torch.float64) * w.v_descale
    return k, v


def contiguous_kv(w: synth.Workload, b: int, kpool=None, vpool=None):
    """K and V of sequence b as contiguous [L, Hkv, D] float64, gathered with
    one fancy-index per tensor (no per-key loop)."""
    if kpool is None:
        kpool, vpool = decoded_pools(w)
    L = int(w.seq_lens[b])
    j = torch.arange(L)
    phys = w.page_table[b].to(torch.int64)[j // w.page_size]
    slot = j % w.page_size
    return kpool[phys, slot], vpool[phys, slot]


def query_values(w: synth.Workload) -> torch.Tensor:
    """Queries as float64, decoded with torch's own casts (E4M3 codes times
    q_descale for fp8 queries)."""
    if w.q_dtype == "fp8_e4m3":
        return w.q.view(torch.float8_e4m3fn).to(torch.float64) * w.q_descale
    return w.q.to(torch.float64)


def library_attention(w: synth.Workload, causal=None, scale=None):
    """Attention through torch's CPU flash-attention operator in float64.

    Each sequence's K/V is gathered to a contiguous layout, KV heads are
    expanded to query heads with repeat_interleave (contiguous groups), and
    the causal mask is the bottom-right aligned one (query i of a q_len chunk
    sees keys j <= L - q_len + i).  Returns O [T, Hq, D] and LSE [T, Hq].
    """
    causal = w.causal if causal is None else causal
    scale = w.scale if scale is None else scale
    kpool, vpool = decoded_pools(w)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_q_lens.numpy()
    T, Hq, D = w.q.shape
    out = torch.zeros(T, Hq, D, dtype=torch.float64)
    lse = torch.full((T, Hq), -math.inf, dtype=torch.float64)
    op = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu
    for b in range(w.num_seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        ql, L = hi - lo, int(w.seq_lens[b])
        if ql == 0:
            continue
        k, v = contiguous_kv(w, b, kpool, vpool)                   # [L, Hkv, D]
        qb = query_values(w)[lo:hi].permute(1, 0, 2)[None]          # [1, Hq, ql, D]
        kb = k.permute(1, 0, 2).repeat_interleave(G, dim=0)[None].contiguous()
        vb = v.permute(1, 0, 2).repeat_interleave(G, dim=0)[None].contiguous()
        if causal and ql == L:
            o, l = op(qb, kb, vb, 0.0, True, scale=scale)
        else:
            i = torch.arange(ql)[:, None]
            j = torch.arange(L)[None, :]
            vis = (j <= (L - ql + i)) if causal else torch.ones(ql, L, dtype=torch.bool)
            mask = torch.where(vis, 0.0, -math.inf).to(torch.float64)
            o, l = op(qb, kb, vb, 0.0, False, attn_mask=mask, scale=scale)
        out[lo:hi] = o[0].permute(1, 0, 2)
        lse[lo:hi] = l[0].permute(1, 0)
    return out.numpy(), lse.numpy()


def random_workload(seed: int, *, B=None, D=None, page=None, G=None, Hkv=None,
                    kv_dtype="bf16", causal=True, max_len=80, decode=False,
                    poison=True, q_dtype="bf16") -> synth.Workload:
    """A small random workload (varying lengths, chunked prefill and decode rows)."""
    rng = np.random.default_rng(seed)
    B = B if B is not None else int(rng.integers(1, 5))
    D = D if D is not None else int(rng.choice([64, 128, 256]))
    page = page if page is not None else int(rng.choice([16, 32, 64, 128]))
    G = G if G is not None else int(rng.choice([1, 2, 4, 8]))
    Hkv = Hkv if Hkv is not None else int(rng.choice([1, 2, 3]))
    L = rng.integers(1, max_len + 1, size=B)
    if decode:
        ql = np.ones(B, dtype=np.int64)
    else:
        ql = np.array([int(rng.integers(0, l + 1)) if rng.random() < 0.5 else int(l)
                       for l in L])
        ql[ql == 0] = np.minimum(1, L[ql == 0])
    return synth.build(name="random%d" % seed, seq_lens=L, q_lens=ql,
                       num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=page,
                       seed=1000 + seed, kv_dtype=kv_dtype, causal=causal, poison=poison,
                       threads=1, q_dtype=q_dtype)
