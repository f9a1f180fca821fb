"""Seeded synthetic inputs for paged-KV GQA attention.

This module draws the inputs that both the HIP library and the fp64 oracle are
run on.  It holds no attention arithmetic: only random numbers, page
assignment, NaN poisoning of slots that must never be read, and the fp8
quantisation that turns bf16 K/V into the stored fp8 cache.

Recipe (one seed per workload):
  * values: torch's CPU normal generator, N(0, 1) in fp32, rounded to bf16
    (round-to-nearest-even).  Large pools are drawn in fixed chunks, chunk i
    from its own generator seeded (seed, stream, i), so the bytes do not depend
    on the thread count.
  * lengths: integers uniform on an inclusive range, from a seeded generator.
  * pages: pool size P = sum_b ceil(L_b / page) + 1 (one poison page) unless the
    workload fixes P; a seeded random permutation of the P physical pages is
    handed out in (sequence, logical page) order; page-table columns at or past
    ceil(L_b / page) point at the poison page.
  * poison: slots past L_b in a sequence's last page, every unused page and the
    poison page hold NaN (bf16 0x7FC0, fp8 0x7F) in both K and V, so any read
    of a slot the definition excludes shows up in the output.
  * fp8 KV: K and V are drawn in bf16 as above, the per-tensor amax over live
    slots gives descale = amax / 448 (fp32), and each value is stored as
    e4m3(clamp(x / descale, -448, 448)) with round-to-nearest-even (torch's
    float8_e4m3fn cast), i.e. saturating quantisation.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0
FP8_NAN_BYTE = 0x7F
_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str              # "bf16" or "fp8_e4m3"
    causal: bool
    scale: float
    q: torch.Tensor            # bf16 [T, Hq, D]
    k_pool: torch.Tensor       # bf16 or uint8 (fp8 bytes) [P, page, Hkv, D]
    v_pool: torch.Tensor
    page_table: torch.Tensor   # int32 [B, row_stride]; first pt_cols columns logical
    pt_cols: int
    cu_q_lens: torch.Tensor    # int32 [B+1]
    seq_lens: torch.Tensor     # int32 [B]
    k_descale: float = 1.0
    v_descale: float = 1.0
    poison_page: int = -1
    softcap: float = 0.0         # > 0: scores s -> softcap * tanh(s / softcap)
    q_dtype: str = "bf16"        # or "fp8_e4m3": q holds E4M3 codes (uint8), value = code * q_descale
    q_descale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        cu = self.cu_q_lens.numpy().astype(np.int64)
        return cu[1:] - cu[:-1]

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    def visible_pairs(self) -> int:
        """sum over query rows and query heads of the visible key count."""
        L = self.seq_lens.numpy().astype(np.int64)
        ql = self.q_lens
        tot = 0
        for Lb, qb in zip(L, ql):
            if self.causal:
                # rows i = 0..qb-1 see L - qb + i + 1 keys
                tot += qb * (Lb - qb) + qb * (qb + 1) // 2
            else:
                tot += qb * Lb
        return int(tot) * self.num_q_heads

    def kv_bytes(self) -> int:
        """live K and V bytes, each live (token, kv head) row read once."""
        e = 2 if self.kv_dtype == "bf16" else 1
        return int(self.seq_lens.numpy().astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * 2 * e

    def flops(self) -> int:
        """4 * D per visible (row, key) pair: q.k and p.v, 2 flops per mac."""
        return 4 * self.head_dim * self.visible_pairs()

    def qo_bytes(self) -> int:
        """Q read once (1 byte an element for E4M3 codes, else 2) and bf16 O written once."""
        qe = 1 if self.q_dtype == "fp8_e4m3" else 2
        return self.total_q * self.num_q_heads * self.head_dim * (qe + 2)


def _mix(*xs: int) -> int:
    """SplitMix64 finaliser over a tuple of integers: per-chunk seeds."""
    z = 0x9E3779B97F4A7C15
    for x in xs:
        z = (z + (x & 0xFFFFFFFFFFFFFFFF) + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        z ^= z >> 31
    return z & 0x7FFFFFFFFFFFFFFF


def normal_bf16(n: int, seed: int, stream: int, threads: int = 8) -> torch.Tensor:
    """n bf16 values ~ N(0,1), deterministic in (seed, stream)."""
    out = torch.empty(n, dtype=torch.bfloat16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i: int) -> None:
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = torch.Generator().manual_seed(_mix(seed, stream, i))
        out[lo:hi] = torch.randn(hi - lo, generator=g, dtype=torch.float32).to(torch.bfloat16)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with _cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def uniform_int(lo: int, hi: int, n: int, seed: int, stream: int) -> np.ndarray:
    """n integers uniform on the inclusive range [lo, hi]."""
    g = torch.Generator().manual_seed(_mix(seed, stream))
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).numpy()


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    g = torch.Generator().manual_seed(_mix(seed, stream))
    return torch.randperm(n, generator=g).numpy().astype(np.int64)


def quantize_e4m3(x: torch.Tensor, descale: float) -> torch.Tensor:
    """bf16/fp32 tensor -> fp8 e4m3 bytes of clamp(x / descale, +-448), RNE."""
    y = (x.to(torch.float32) / torch.tensor(descale, dtype=torch.float32)).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def build(*, name: str, seq_lens: Sequence[int], q_lens: Sequence[int],
          num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
          seed: int, kv_dtype: str = "bf16", causal: bool = True,
          scale: Optional[float] = None, pt_cols: Optional[int] = None,
          pt_row_stride: Optional[int] = None, num_pages: Optional[int] = None,
          poison: bool = True, threads: int = 8, q_dtype: str = "bf16") -> Workload:
    """Generic builder; every named workload below is a call of this."""
    L = np.asarray(seq_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    B = L.size
    assert ql.size == B and np.all(ql >= 0) and np.all(ql <= L)
    D, Hq, Hkv, page = head_dim, num_q_heads, num_kv_heads, page_size
    assert Hq % Hkv == 0
    pages_per_seq = (L + page - 1) // page
    need = int(pages_per_seq.sum())
    if pt_cols is None:
        pt_cols = int(max(1, pages_per_seq.max() if B else 1))
    assert pt_cols >= (pages_per_seq.max() if B else 0)
    row_stride = pt_row_stride if pt_row_stride is not None else pt_cols
    assert row_stride >= pt_cols
    P = num_pages if num_pages is not None else need + 1
    assert P >= need + 1, "pool must hold every live page plus the poison page"

    perm = permutation(P, seed, 1)
    pt = np.empty((B, row_stride), dtype=np.int32)
    poison_page = int(perm[need])
    pt[:, :] = poison_page
    cursor = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        pt[b, :n] = perm[cursor:cursor + n]
        cursor += n

    # live-slot mask over the pool, [P, page]
    live = np.zeros((P, page), dtype=bool)
    for b in range(B):
        for p in range(int(pages_per_seq[b])):
            cnt = min(page, int(L[b]) - p * page)
            live[pt[b, p], :cnt] = True
    live_t = torch.from_numpy(live)

    T = int(ql.sum())
    q = normal_bf16(T * Hq * D, seed, 2, threads).view(T, Hq, D)
    pool_elems = P * page * Hkv * D
    k = normal_bf16(pool_elems, seed, 3, threads).view(P, page, Hkv, D)
    v = normal_bf16(pool_elems, seed, 4, threads).view(P, page, Hkv, D)

    k_descale = v_descale = 1.0
    if kv_dtype == "bf16":
        if poison:
            nan = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
            dead = ~live_t
            k[dead] = nan
            v[dead] = nan
    elif kv_dtype == "fp8_e4m3":
        def amax(x):
            return float(x[live_t].abs().max().to(torch.float32)) if live.any() else 1.0
        k_descale = float(np.float32(amax(k) / 448.0))
        v_descale = float(np.float32(amax(v) / 448.0))
        k = quantize_e4m3(k, k_descale)
        v = quantize_e4m3(v, v_descale)
        if poison:
            dead = ~live_t
            k[dead] = FP8_NAN_BYTE
            v[dead] = FP8_NAN_BYTE
    else:
        raise ValueError(kv_dtype)

    q_descale = 1.0
    if q_dtype == "fp8_e4m3":
        # the same per-tensor quantisation as the cache: descale = amax / 448
        amax_q = float(q.abs().max().to(torch.float32)) if q.numel() else 1.0
        q_descale = float(np.float32(amax_q / 448.0)) if amax_q > 0 else 1.0
        q = quantize_e4m3(q, q_descale)
    elif q_dtype != "bf16":
        raise ValueError(q_dtype)

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    page_size=page, kv_dtype=kv_dtype, causal=causal,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
                    q=q, k_pool=k, v_pool=v,
                    page_table=torch.from_numpy(pt), pt_cols=int(pt_cols),
                    cu_q_lens=torch.from_numpy(cu),
                    seq_lens=torch.from_numpy(L.astype(np.int32)),
                    k_descale=k_descale, v_descale=v_descale, poison_page=poison_page,
                    q_dtype=q_dtype, q_descale=q_descale)


# ---------------------------------------------------------------------------
# The five named workloads.  Shapes follow the attention geometry the pages
# measure on: Llama-3.1-8B heads 32/8 hd128 decode and prefill (vLLM PR
# #48156, kernel micro-benchmark table), the 24B-class 1000-token-input
# serving run (vLLM PR #16828, "Further benchmarking"), and the widest
# decode geometry of TensorRT-LLM PR #17399 ("Integration and supported
# scope": page 128, head dim 256, GQA ratio 32) with an fp8 cache.
# ---------------------------------------------------------------------------

def tiny_mixed(seed: int = 1, **kw) -> Workload:
    """B=2, Hq/Hkv 4/2, D 64, page 16: a 37-token causal prefill (L=37) and a
    decode row (L=50), 16-page pool, page table [2, 4]."""
    return build(name="tiny_mixed", seq_lens=[37, 50], q_lens=[37, 1], num_q_heads=4,
                 num_kv_heads=2, head_dim=64, page_size=16, seed=seed, pt_cols=4,
                 num_pages=16, scale=1.0 / 8.0, **kw)


def decode_llama8b(seed: int = 2, **kw) -> Workload:
    """B=256 decode rows, Hq/Hkv 32/8, D 128, page 16, L ~ U[1024, 2048]."""
    L = uniform_int(1024, 2048, 256, seed, 0)
    return build(name="decode_llama8b", seq_lens=L, q_lens=[1] * 256, num_q_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=16, seed=seed, pt_cols=128, **kw)


def prefill_causal(seed: int = 3, **kw) -> Workload:
    """16 causal prefills, q_len = L ~ U[512, 4096], Hq/Hkv 32/8, D 128, page 64."""
    L = uniform_int(512, 4096, 16, seed, 0)
    return build(name="prefill_causal", seq_lens=L, q_lens=L, num_q_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=64, seed=seed, pt_cols=64, **kw)


def prefill_causal_d256(seed: int = 8, **kw) -> Workload:
    """16 causal prefills, q_len = L ~ U[512, 4096], Hq/Hkv 16/4, D 256, page 64:
    the context head dim 256 of the supported scope, at the flops of
    prefill_causal (half the heads, twice the head dim)."""
    L = uniform_int(512, 4096, 16, seed, 0)
    return build(name="prefill_causal_d256", seq_lens=L, q_lens=L, num_q_heads=16,
                 num_kv_heads=4, head_dim=256, page_size=64, seed=seed, pt_cols=64, **kw)


def mixed_24b(seed: int = 4, shuffle: bool = False, **kw) -> Workload:
    """8 prefill chunks of 1000 new tokens on 0..1000 cached tokens, then 248
    decode rows with L ~ U[1000, 2000]; Hq/Hkv 32/8, D 128, page 16."""
    cached = uniform_int(0, 1000, 8, seed, 0)
    dec = uniform_int(1000, 2000, 248, seed, 5)
    L = np.concatenate([cached + 1000, dec])
    ql = np.concatenate([np.full(8, 1000), np.ones(248, dtype=np.int64)])
    if shuffle:
        order = permutation(256, seed, 6)
        L, ql = L[order], ql[order]
    return build(name="mixed_24b" + ("_shuffled" if shuffle else ""), seq_lens=L, q_lens=ql,
                 num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, seed=seed,
                 pt_cols=125, **kw)


def decode_fp8_long(seed: int = 5, **kw) -> Workload:
    """B=64 decode rows, Hq/Hkv 64/2 (ratio 32), D 256, page 128,
    L ~ U[4096, 32768], fp8 e4m3 K/V with per-tensor descale."""
    L = uniform_int(4096, 32768, 64, seed, 0)
    return build(name="decode_fp8_long", seq_lens=L, q_lens=[1] * 64, num_q_heads=64,
                 num_kv_heads=2, head_dim=256, page_size=128, seed=seed, pt_cols=256,
                 kv_dtype="fp8_e4m3", **kw)


# ---------------------------------------------------------------------------
# MLA decode workloads (DeepSeek-style latent cache: one logical KV head, a
# 576-wide cached row = 512 latent values then 64 RoPE key values; the latent
# part is also the value).  The measured MLA run of TensorRT-LLM PR #17399
# (results table: DeepSeek-V3-Lite, page size 32, 1024-token inputs and
# outputs, concurrency 64) fixes B = 64 decode rows, page 32 and lengths from
# 1025 to 2048; its head count is not given, so both ends of the supported
# range are built: 16 query heads (a Lite-sized model) and 128 (the maximum).
# ---------------------------------------------------------------------------

MLA_LATENT = 512
MLA_ROPE = 64


@dataclasses.dataclass
class MlaWorkload:
    name: str
    num_q_heads: int
    page_size: int
    scale: float
    q: torch.Tensor            # bf16 [B, Hq, 576]
    kv: torch.Tensor           # bf16 [P, page, 576]
    page_table: torch.Tensor   # int32 [B, row_stride]
    pt_cols: int
    seq_lens: torch.Tensor     # int32 [B]
    poison_page: int = -1
    softcap: float = 0.0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    def kv_bytes(self) -> int:
        """Cached bytes read once: every live row, 576 bf16 values."""
        return int(self.seq_lens.to(torch.int64).sum()) * (MLA_LATENT + MLA_ROPE) * 2

    def qo_bytes(self) -> int:
        return self.num_seqs * self.num_q_heads * (MLA_LATENT + MLA_ROPE + MLA_LATENT) * 2

    def flops(self) -> int:
        """2 (576 + 512) flops per (query head, key) pair."""
        return int(self.seq_lens.to(torch.int64).sum()) * self.num_q_heads * 2 * (
            MLA_LATENT + MLA_ROPE + MLA_LATENT)


def build_mla(*, name: str, seq_lens: Sequence[int], num_q_heads: int, page_size: int, seed: int,
              scale: Optional[float] = None, pt_cols: Optional[int] = None,
              pt_row_stride: Optional[int] = None, poison: bool = True,
              threads: int = 8) -> MlaWorkload:
    """Latent cache and queries with the same page handling as build():
    seeded page permutation, a poison page for unused columns, NaN in dead slots."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B, page, Dk = L.size, page_size, MLA_LATENT + MLA_ROPE
    pages_per_seq = (L + page - 1) // page
    need = int(pages_per_seq.sum())
    if pt_cols is None:
        pt_cols = int(max(1, pages_per_seq.max() if B else 1))
    row_stride = pt_row_stride if pt_row_stride is not None else pt_cols
    P = need + 1
    perm = permutation(P, seed, 1)
    pt = np.empty((B, row_stride), dtype=np.int32)
    poison_page = int(perm[need])
    pt[:, :] = poison_page
    cursor = 0
    live = np.zeros((P, page), dtype=bool)
    for b in range(B):
        n = int(pages_per_seq[b])
        pt[b, :n] = perm[cursor:cursor + n]
        cursor += n
        for p in range(n):
            live[pt[b, p], :min(page, int(L[b]) - p * page)] = True
    q = normal_bf16(B * num_q_heads * Dk, seed, 2, threads).view(B, num_q_heads, Dk)
    kv = normal_bf16(P * page * Dk, seed, 3, threads).view(P, page, Dk)
    if poison:
        kv[~torch.from_numpy(live)] = torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
    return MlaWorkload(name=name, num_q_heads=num_q_heads, page_size=page,
                       scale=float(scale if scale is not None else 1.0 / math.sqrt(Dk)),
                       q=q, kv=kv, page_table=torch.from_numpy(pt), pt_cols=int(pt_cols),
                       seq_lens=torch.from_numpy(L.astype(np.int32)), poison_page=poison_page)


def mla_decode_h16(seed: int = 6, **kw) -> MlaWorkload:
    """B=64 MLA decode rows, 16 query heads, page 32, L ~ U[1025, 2048]."""
    L = uniform_int(1025, 2048, 64, seed, 0)
    return build_mla(name="mla_decode_h16", seq_lens=L, num_q_heads=16, page_size=32, seed=seed,
                     pt_cols=64, **kw)


def mla_decode_h128(seed: int = 7, **kw) -> MlaWorkload:
    """B=64 MLA decode rows, 128 query heads, page 32, L ~ U[1025, 2048]."""
    L = uniform_int(1025, 2048, 64, seed, 0)
    return build_mla(name="mla_decode_h128", seq_lens=L, num_q_heads=128, page_size=32, seed=seed,
                     pt_cols=64, **kw)


WORKLOADS = {
    "tiny_mixed": tiny_mixed,
    "decode_llama8b": decode_llama8b,
    "prefill_causal": prefill_causal,
    "prefill_causal_d256": prefill_causal_d256,
    "mixed_24b": mixed_24b,
    "decode_fp8_long": decode_fp8_long,
    "mla_decode_h16": mla_decode_h16,
    "mla_decode_h128": mla_decode_h128,
}


def sample_rows(w: Workload, per_seq: int = 3, heads: int = 4, seed: int = 99) -> List[int]:
    """A deterministic sample of flat (t*Hq + h) rows: per sequence its first
    and last query token plus random ones, each with a few query heads spread
    over distinct KV heads."""
    rng = np.random.default_rng(seed)
    cu = w.cu_q_lens.numpy()
    Hq = w.num_q_heads
    rows = []
    for b in range(w.num_seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        toks = {lo, hi - 1}
        for _ in range(max(0, per_seq - 2)):
            toks.add(int(rng.integers(lo, hi)))
        for t in sorted(toks):
            hs = set(int(x) for x in rng.choice(Hq, size=min(heads, Hq), replace=False))
            for h in sorted(hs):
                rows.append(t * Hq + h)
    return rows
