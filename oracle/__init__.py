"""fp64 CPU oracle for paged-KV grouped-query attention.

TEST INFRASTRUCTURE ONLY: the parity reference for the HIP kernels.  Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with
``paged_kv_gqa_attention_amd`` and never imports it.

The arithmetic lives in ``pa_oracle.c`` (plain C99, double precision, one row
at a time).  This module only builds that file with gcc and marshals numpy
arrays into it.  See ``pa_oracle.h`` for the definition being computed and the
passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
Q_BF16 = 0
Q_FP8_E4M3 = 1


def compile_source(src: str, out: str) -> str:
    """gcc a C source of the oracle into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile pa_oracle.c with gcc into oracle/libpa_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("pt_cols", ctypes.c_int32),
        ("pt_row_stride", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
        ("q_stride_t", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("k_descale", ctypes.c_double),
        ("v_descale", ctypes.c_double),
        ("softcap", ctypes.c_double),
        ("q_dtype", ctypes.c_int32),
        ("q_descale", ctypes.c_double),
    ]


class MlaProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("pt_cols", ctypes.c_int32),
        ("pt_row_stride", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
        ("q_stride_t", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("softcap", ctypes.c_double),
    ]


_lib = None


def load(path: str):
    """Open a compiled oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.pao_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.pao_bf16_to_double.restype = ctypes.c_double
    L.pao_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
    L.pao_fp8_e4m3_to_double.restype = ctypes.c_double
    L.pao_attention.argtypes = [ctypes.POINTER(Problem), vp, vp, vp, vp, vp, vp,
                                ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_int64,
                                vp, vp, ctypes.c_int]
    L.pao_attention.restype = ctypes.c_int
    L.pao_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                            vp, vp, vp, vp]
    L.pao_merge.restype = ctypes.c_int
    L.pao_fp8_e4m3_encode.argtypes = [ctypes.c_double]
    L.pao_fp8_e4m3_encode.restype = ctypes.c_uint8
    L.pao_append.argtypes = [ctypes.POINTER(Problem), vp, vp, ctypes.c_int64, vp, vp, vp, vp, vp]
    L.pao_append.restype = ctypes.c_int
    L.pao_mla_decode.argtypes = [ctypes.POINTER(MlaProblem), vp, vp, vp, vp, vp, ctypes.c_int64,
                                 vp, vp, ctypes.c_int]
    L.pao_mla_decode.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        build(force=False)                  # compiles when missing or older than the source
        _lib = load(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def bf16_to_double(bits: int) -> float:
    return lib().pao_bf16_to_double(int(bits))


def fp8_e4m3_to_double(byte: int) -> float:
    return lib().pao_fp8_e4m3_to_double(int(byte))


def attention(*, q_bits: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
              page_table: np.ndarray, cu_q_lens: np.ndarray, seq_lens: np.ndarray,
              num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
              scale: float, causal: bool = True, kv_dtype: int = KV_BF16,
              k_descale: float = 1.0, v_descale: float = 1.0,
              rows: Optional[Sequence[int]] = None,
              key_begin: int = 0, key_end: int = -1,
              q_stride_t: int = 0, kv_page_stride: int = 0,
              pt_cols: Optional[int] = None, threads: int = 0, softcap: float = 0.0,
              q_dtype: int = Q_BF16, q_descale: float = 1.0):
    """Reference attention in fp64.

    q_bits   : uint16 bf16 bit patterns, [T, Hq, D] (or a flat buffer with
               ``q_stride_t`` elements between tokens); uint8 E4M3 codes when
               ``q_dtype`` is Q_FP8_E4M3 (value = code * q_descale)
    k_pool, v_pool : uint16 (bf16 bits) or uint8 (fp8 e4m3 bytes),
               [P, page, Hkv, D] (or flat with ``kv_page_stride``)
    page_table : int32 [B, row_stride]; the first ``pt_cols`` columns (default:
               all) are logical pages, the rest is padding that is never read
    rows     : None for every (t, h); else flat indices t*Hq + h
    Returns (out, lse): fp64 [T, Hq, D] and [T, Hq] when rows is None,
    else [len(rows), D] and [len(rows)].
    """
    page_table = _c(page_table, np.int32)
    if page_table.ndim != 2:
        raise OracleError("page_table must be 2-D [B, row_stride]")
    cu_q_lens = _c(cu_q_lens, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    q_bits = _c(q_bits, np.uint16 if q_dtype == Q_BF16 else np.uint8)
    kv_np = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    k_pool = _c(k_pool, kv_np)
    v_pool = _c(v_pool, kv_np)
    B = seq_lens.shape[0]
    D = head_dim
    per_page = kv_page_stride if kv_page_stride else page_size * num_kv_heads * D
    P = k_pool.size // per_page
    pr = Problem(num_seqs=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=D, page_size=page_size, num_pages=P,
                 pt_cols=page_table.shape[1] if pt_cols is None else pt_cols,
                 pt_row_stride=page_table.shape[1],
                 kv_page_stride=kv_page_stride, q_stride_t=q_stride_t,
                 kv_dtype=kv_dtype, causal=1 if causal else 0, scale=scale,
                 k_descale=k_descale, v_descale=v_descale, softcap=softcap,
                 q_dtype=q_dtype, q_descale=q_descale)
    T = int(cu_q_lens[B]) if B else 0
    if rows is None:
        rows_arr = None
        n = T * num_q_heads
        out = np.zeros((T, num_q_heads, D), np.float64)
        lse = np.zeros((T, num_q_heads), np.float64)
    else:
        rows_arr = _c(rows, np.int64)
        n = rows_arr.size
        out = np.zeros((n, D), np.float64)
        lse = np.zeros((n,), np.float64)
    rc = lib().pao_attention(ctypes.byref(pr), _ptr(q_bits), _ptr(k_pool), _ptr(v_pool),
                             _ptr(page_table), _ptr(cu_q_lens), _ptr(seq_lens),
                             int(key_begin), int(key_end), _ptr(rows_arr), int(n),
                             _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise OracleError("pao_attention failed with code %d" % rc)
    return out, lse


def workload_arrays(w):
    """numpy views of a workload object (anything with the attributes of the
    seeded workloads: q, k_pool, v_pool as torch CPU tensors, kv_dtype and
    q_dtype names): q as bf16 bits or E4M3 codes, K/V pools as bf16 bits or
    fp8 bytes.  Marshalling only."""
    import torch
    if w.q.dtype == torch.uint8:                      # fp8 queries: E4M3 codes
        q = w.q.contiguous().numpy()
    else:
        q = w.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    if w.kv_dtype == "bf16":
        k = w.k_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
        v = w.v_pool.contiguous().view(torch.int16).numpy().view(np.uint16)
    else:
        k = w.k_pool.contiguous().numpy()
        v = w.v_pool.contiguous().numpy()
    return q, k, v


def attention_workload(w, rows=None, key_begin=0, key_end=-1, causal=None, scale=None,
                       threads=0, softcap=None):
    """attention() over a workload object's tensors and metadata (argument
    marshalling only; see workload_arrays)."""
    q, k, v = workload_arrays(w)
    return attention(
        q_bits=q, k_pool=k, v_pool=v, page_table=w.page_table.numpy(),
        cu_q_lens=w.cu_q_lens.numpy(), seq_lens=w.seq_lens.numpy(),
        num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
        page_size=w.page_size, scale=w.scale if scale is None else scale,
        causal=w.causal if causal is None else causal,
        kv_dtype=KV_BF16 if w.kv_dtype == "bf16" else KV_FP8_E4M3,
        k_descale=w.k_descale, v_descale=w.v_descale, rows=rows,
        key_begin=key_begin, key_end=key_end, pt_cols=w.pt_cols, threads=threads,
        softcap=w.softcap if softcap is None else softcap,
        q_dtype=Q_FP8_E4M3 if w.q_dtype == "fp8_e4m3" else Q_BF16,
        q_descale=w.q_descale)


def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine partials over disjoint key windows: o_parts [S, n, D], lse_parts [S, n]."""
    o_parts = _c(o_parts, np.float64)
    lse_parts = _c(lse_parts, np.float64)
    S, n, D = o_parts.shape
    o = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = lib().pao_merge(S, n, D, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse))
    if rc != 0:
        raise OracleError("pao_merge failed with code %d" % rc)
    return o, lse


def fp8_e4m3_encode(x: float) -> int:
    """Nearest finite E4M3 code to x (ties to an even mantissa), saturating; NaN keeps its sign."""
    return int(lib().pao_fp8_e4m3_encode(float(x)))


def append(*, k_new: np.ndarray, v_new: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
           page_table: np.ndarray, cu_new: np.ndarray, seq_lens: np.ndarray,
           num_kv_heads: int, head_dim: int, page_size: int, kv_dtype: int = KV_BF16,
           k_descale: float = 1.0, v_descale: float = 1.0, new_stride_t: int = 0,
           kv_page_stride: int = 0, pt_cols: Optional[int] = None):
    """KV-cache append (see pa_oracle.h).  Returns updated copies of the pools.

    k_new, v_new : uint16 bf16 bits [T_new, Hkv, D] (or flat with new_stride_t)
    k_pool, v_pool : uint16 (bf16 bits) or uint8 (fp8 codes), [P, page, Hkv, D]
    cu_new   : int32 [B+1] offsets of each sequence's new tokens
    seq_lens : int32 [B] lengths after the append
    """
    page_table = _c(page_table, np.int32)
    cu_new = _c(cu_new, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    kv_np = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    k_out = np.array(k_pool, dtype=kv_np, copy=True, order="C")
    v_out = np.array(v_pool, dtype=kv_np, copy=True, order="C")
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    per_page = kv_page_stride if kv_page_stride else page_size * num_kv_heads * head_dim
    pr = Problem(num_seqs=seq_lens.shape[0], num_q_heads=num_kv_heads,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                 num_pages=k_out.size // per_page,
                 pt_cols=page_table.shape[1] if pt_cols is None else pt_cols,
                 pt_row_stride=page_table.shape[1], kv_page_stride=kv_page_stride,
                 q_stride_t=0, kv_dtype=kv_dtype, causal=1, scale=1.0,
                 k_descale=k_descale, v_descale=v_descale)
    rc = lib().pao_append(ctypes.byref(pr), _ptr(k_new), _ptr(v_new), int(new_stride_t),
                          _ptr(page_table), _ptr(cu_new), _ptr(seq_lens), _ptr(k_out), _ptr(v_out))
    if rc != 0:
        raise OracleError("pao_append failed with code %d" % rc)
    return k_out, v_out


def mla_decode(*, q_bits: np.ndarray, kv_cache: np.ndarray, page_table: np.ndarray,
               seq_lens: np.ndarray, num_q_heads: int, page_size: int, scale: float,
               d_latent: int = 512, d_rope: int = 64, softcap: float = 0.0,
               rows: Optional[Sequence[int]] = None, q_stride_t: int = 0,
               kv_page_stride: int = 0, pt_cols: Optional[int] = None, threads: int = 0):
    """MLA decode in fp64 (see pa_oracle.h).

    q_bits   : uint16 bf16 bits [B, Hq, d_latent + d_rope]
    kv_cache : uint16 bf16 bits [P, page, d_latent + d_rope]
    Returns (out, lse): [B, Hq, d_latent] and [B, Hq] when rows is None, else
    [len(rows), d_latent] and [len(rows)] for flat rows b*Hq + h.
    """
    page_table = _c(page_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    q_bits = _c(q_bits, np.uint16)
    kv_cache = _c(kv_cache, np.uint16)
    B = seq_lens.shape[0]
    Dk = d_latent + d_rope
    per_page = kv_page_stride if kv_page_stride else page_size * Dk
    pr = MlaProblem(num_seqs=B, num_q_heads=num_q_heads, d_latent=d_latent, d_rope=d_rope,
                    page_size=page_size, num_pages=kv_cache.size // per_page,
                    pt_cols=page_table.shape[1] if pt_cols is None else pt_cols,
                    pt_row_stride=page_table.shape[1], kv_page_stride=kv_page_stride,
                    q_stride_t=q_stride_t, scale=scale, softcap=softcap)
    if rows is None:
        rows_arr = None
        n = B * num_q_heads
    else:
        rows_arr = _c(np.asarray(rows), np.int64)
        n = rows_arr.shape[0]
    out = np.zeros((n, d_latent), np.float64)
    lse = np.zeros(n, np.float64)
    rc = lib().pao_mla_decode(ctypes.byref(pr), _ptr(q_bits), _ptr(kv_cache), _ptr(page_table),
                              _ptr(seq_lens), _ptr(rows_arr), int(n), _ptr(out), _ptr(lse),
                              int(threads))
    if rc != 0:
        raise OracleError("pao_mla_decode failed with code %d" % rc)
    if rows is None:
        return out.reshape(B, num_q_heads, d_latent), lse.reshape(B, num_q_heads)
    return out, lse
