"""ctypes binding of libpa.so (the C ABI declared in include/pa.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels of libpa.so.  torch is used for device memory and the current HIP
stream.  The functions keep the C names:

    pa_plan(desc) -> plan            pa_workspace_bytes(plan) -> int
    pa_plan_get_info(plan) -> info   pa_plan_destroy(plan)
    pa_run_prefill / pa_run_decode / pa_run_mixed(plan, args, stream) -> None
    pa_run_decode_static(plan, args, stream) -> None
    pa_run_append(plan, append_args, stream) -> None
    pa_mla_plan(mla_desc) -> plan    pa_mla_workspace_bytes(plan) -> int
    pa_mla_num_splits(plan) -> int   pa_mla_plan_destroy(plan)
    pa_run_mla_decode(plan, mla_args, stream) -> None
    pa_status_str(code) -> str

Errors are raised as ``PaError`` carrying the status code.  If libpa.so has not
been built, the first call raises ``PaLibraryMissing``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_SCRATCH = -5
PA_STATIC_SCRATCH_BYTES = 32 << 20     # include/pa.h

PA_KV_BF16 = 0
PA_KV_FP8_E4M3 = 1
PA_Q_BF16 = 0
PA_Q_FP8_E4M3 = 1

EXPORTS = ("pa_plan", "pa_workspace_bytes", "pa_plan_get_info", "pa_run_prefill",
           "pa_run_decode", "pa_run_mixed", "pa_run_append", "pa_plan_destroy", "pa_status_str",
           "pa_mla_plan", "pa_mla_workspace_bytes", "pa_mla_num_splits", "pa_run_mla_decode",
           "pa_mla_plan_destroy", "pa_check_metadata", "pa_run_decode_static",
           "pa_calibrate_mfma", "pa_calibrate_mfma_flops")

PA_CHECK_PAGE_ID = 1
PA_CHECK_Q_LEN = 2
PA_CHECK_SEQ_LEN = 4
PA_CHECK_CU_Q_LENS = 8


class PaLibraryMissing(RuntimeError):
    pass


class PaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (%d)" % (where, pa_status_str(code), code))


class pa_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_table_cols", ctypes.c_int32),
        ("page_table_row_stride", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
        ("max_total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
    ]


class pa_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_stride_t", ctypes.c_int64),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("cu_q_lens", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("o_stride_t", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("softcap", ctypes.c_float),
        ("q_descale", ctypes.c_void_p),
    ]


class pa_plan_info(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32),
        ("split_keys", ctypes.c_int32),
        ("q_block_tokens", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("mixed_q_block_tokens", ctypes.c_int32),
        ("balanced_workgroups", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("queue_workgroups", ctypes.c_int32),
    ]


class pa_append_args(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("new_stride_t", ctypes.c_int64),
        ("cu_new", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
    ]


class pa_mla_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_table_cols", ctypes.c_int32),
        ("page_table_row_stride", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
        ("max_seq_len", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
    ]


class pa_mla_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_stride_t", ctypes.c_int64),
        ("kv_cache", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("o_stride_t", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib():
    """Open libpa.so (once) and declare the signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PaLibraryMissing(
                "libpa.so not found at %s; build it with `python -m "
                "paged_kv_gqa_attention_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.pa_plan.argtypes = [ctypes.POINTER(pa_desc), ctypes.POINTER(vp)]
        L.pa_plan.restype = ctypes.c_int
        L.pa_workspace_bytes.argtypes = [vp]
        L.pa_workspace_bytes.restype = ctypes.c_size_t
        L.pa_plan_get_info.argtypes = [vp, ctypes.POINTER(pa_plan_info)]
        L.pa_plan_get_info.restype = ctypes.c_int
        for name in ("pa_run_prefill", "pa_run_decode", "pa_run_mixed", "pa_run_decode_static"):
            f = getattr(L, name)
            f.argtypes = [vp, ctypes.POINTER(pa_args), vp]
            f.restype = ctypes.c_int
        L.pa_run_append.argtypes = [vp, ctypes.POINTER(pa_append_args), vp]
        L.pa_run_append.restype = ctypes.c_int
        L.pa_plan_destroy.argtypes = [vp]
        L.pa_plan_destroy.restype = None
        L.pa_check_metadata.argtypes = [vp, ctypes.POINTER(pa_args), vp, vp]
        L.pa_check_metadata.restype = ctypes.c_int
        L.pa_status_str.argtypes = [ctypes.c_int]
        L.pa_status_str.restype = ctypes.c_char_p
        L.pa_mla_plan.argtypes = [ctypes.POINTER(pa_mla_desc), ctypes.POINTER(vp)]
        L.pa_mla_plan.restype = ctypes.c_int
        L.pa_mla_workspace_bytes.argtypes = [vp]
        L.pa_mla_workspace_bytes.restype = ctypes.c_size_t
        L.pa_mla_num_splits.argtypes = [vp]
        L.pa_mla_num_splits.restype = ctypes.c_int32
        L.pa_run_mla_decode.argtypes = [vp, ctypes.POINTER(pa_mla_args), vp]
        L.pa_run_mla_decode.restype = ctypes.c_int
        L.pa_mla_plan_destroy.argtypes = [vp]
        L.pa_mla_plan_destroy.restype = None
        L.pa_calibrate_mfma.argtypes = [vp, ctypes.c_int64, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, vp]
        L.pa_calibrate_mfma.restype = ctypes.c_int
        L.pa_calibrate_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.pa_calibrate_mfma_flops.restype = ctypes.c_double
        _lib = L
    return _lib


def pa_status_str(code: int) -> str:
    return lib().pa_status_str(int(code)).decode()


def pa_plan(desc: pa_desc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    rc = lib().pa_plan(ctypes.byref(desc), ctypes.byref(h))
    if rc != PA_OK:
        raise PaError(rc, "pa_plan")
    return h


def pa_workspace_bytes(plan) -> int:
    return int(lib().pa_workspace_bytes(plan))


def pa_plan_get_info(plan) -> pa_plan_info:
    info = pa_plan_info()
    rc = lib().pa_plan_get_info(plan, ctypes.byref(info))
    if rc != PA_OK:
        raise PaError(rc, "pa_plan_get_info")
    return info


def pa_plan_destroy(plan) -> None:
    lib().pa_plan_destroy(plan)


def _run(name: str, plan, args: pa_args, stream) -> None:
    rc = getattr(lib(), name)(plan, ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != PA_OK:
        raise PaError(rc, name)


def pa_run_prefill(plan, args: pa_args, stream) -> None:
    _run("pa_run_prefill", plan, args, stream)


def pa_run_decode(plan, args: pa_args, stream) -> None:
    _run("pa_run_decode", plan, args, stream)


def pa_run_mixed(plan, args: pa_args, stream) -> None:
    _run("pa_run_mixed", plan, args, stream)


def pa_run_decode_static(plan, args: pa_args, stream) -> None:
    """pa_run_decode with the library's static scratch (args' workspace ignored)."""
    _run("pa_run_decode_static", plan, args, stream)


def pa_check_metadata(plan, args: pa_args, flags, stream) -> None:
    """Queue the metadata check; `flags` is a device int32 (tensor or pointer)."""
    fp = _ptr(flags) if hasattr(flags, "data_ptr") else flags
    rc = lib().pa_check_metadata(plan, ctypes.byref(args), ctypes.c_void_p(fp), ctypes.c_void_p(stream))
    if rc != PA_OK:
        raise PaError(rc, "pa_check_metadata")


def pa_run_append(plan, args: "pa_append_args", stream) -> None:
    rc = lib().pa_run_append(plan, ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != PA_OK:
        raise PaError(rc, "pa_run_append")


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def make_desc(*, num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
              page_size: int, num_pages: int, page_table_cols: int,
              page_table_row_stride: Optional[int] = None, kv_page_stride: int = 0,
              max_total_q: int, max_q_len: int, max_seq_len: int = 0,
              kv_dtype: int = PA_KV_BF16, num_splits: int = 0, num_cus: int = 0,
              q_dtype: int = PA_Q_BF16) -> pa_desc:
    return pa_desc(num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                   head_dim=head_dim, page_size=page_size, num_pages=num_pages,
                   page_table_cols=page_table_cols,
                   page_table_row_stride=(page_table_row_stride if page_table_row_stride
                                          is not None else page_table_cols),
                   kv_page_stride=kv_page_stride, max_total_q=max_total_q,
                   max_q_len=max_q_len, max_seq_len=max_seq_len, kv_dtype=kv_dtype,
                   num_splits=num_splits, num_cus=num_cus, q_dtype=q_dtype)


def make_args(*, q, k_pool, v_pool, page_table, cu_q_lens, seq_lens, softmax_scale: float,
              causal: bool, out, lse=None, k_descale=None, v_descale=None, workspace=None,
              q_stride_t: int = 0, o_stride_t: int = 0, softcap: float = 0.0,
              q_descale=None) -> pa_args:
    """Build pa_args from device tensors (no copies, no checks beyond the C side)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return pa_args(q=_ptr(q), q_stride_t=q_stride_t, k_pool=_ptr(k_pool), v_pool=_ptr(v_pool),
                   page_table=_ptr(page_table), cu_q_lens=_ptr(cu_q_lens),
                   seq_lens=_ptr(seq_lens), softmax_scale=float(softmax_scale),
                   causal=1 if causal else 0, k_descale=_ptr(k_descale),
                   v_descale=_ptr(v_descale), out=_ptr(out), o_stride_t=o_stride_t,
                   lse=_ptr(lse), workspace=_ptr(workspace), workspace_bytes=ws_bytes,
                   softcap=float(softcap), q_descale=_ptr(q_descale))


def make_append_args(*, k_new, v_new, cu_new, seq_lens, page_table, k_pool, v_pool,
                     k_descale=None, v_descale=None, new_stride_t: int = 0) -> "pa_append_args":
    """Build pa_append_args from device tensors."""
    return pa_append_args(k_new=_ptr(k_new), v_new=_ptr(v_new), new_stride_t=new_stride_t,
                          cu_new=_ptr(cu_new), seq_lens=_ptr(seq_lens),
                          page_table=_ptr(page_table), k_pool=_ptr(k_pool), v_pool=_ptr(v_pool),
                          k_descale=_ptr(k_descale), v_descale=_ptr(v_descale))


def current_stream() -> int:
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def pa_mla_plan(desc: pa_mla_desc) -> ctypes.c_void_p:
    plan = ctypes.c_void_p()
    rc = lib().pa_mla_plan(ctypes.byref(desc), ctypes.byref(plan))
    if rc != PA_OK:
        raise PaError(rc, "pa_mla_plan")
    return plan


def pa_mla_workspace_bytes(plan) -> int:
    return int(lib().pa_mla_workspace_bytes(plan))


def pa_mla_num_splits(plan) -> int:
    return int(lib().pa_mla_num_splits(plan))


def pa_run_mla_decode(plan, args: pa_mla_args, stream) -> None:
    rc = lib().pa_run_mla_decode(plan, ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != PA_OK:
        raise PaError(rc, "pa_run_mla_decode")


def pa_mla_plan_destroy(plan) -> None:
    lib().pa_mla_plan_destroy(plan)


def make_mla_args(*, q, kv_cache, page_table, seq_lens, softmax_scale: float, out, lse=None,
                  workspace=None, softcap: float = 0.0, q_stride_t: int = 0,
                  o_stride_t: int = 0) -> pa_mla_args:
    """Build pa_mla_args from device tensors."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return pa_mla_args(q=_ptr(q), q_stride_t=q_stride_t, kv_cache=_ptr(kv_cache),
                       page_table=_ptr(page_table), seq_lens=_ptr(seq_lens),
                       softmax_scale=float(softmax_scale), softcap=float(softcap), out=_ptr(out),
                       o_stride_t=o_stride_t, lse=_ptr(lse), workspace=_ptr(workspace),
                       workspace_bytes=ws_bytes)


def pa_calibrate_mfma(operands, sink, num_workgroups: int, iters: int, stream, fp8: bool = False) -> None:
    """MFMA-rate measurement launch (operands: num_workgroups * 32768 16-bit
    words for bf16, 65536 for E4M3; sink: num_workgroups * 256 float32; both
    device tensors)."""
    rc = lib().pa_calibrate_mfma(_ptr(operands), int(operands.numel() * operands.element_size() // 2), _ptr(sink),
                                 int(sink.numel()), int(num_workgroups), int(iters), int(bool(fp8)), stream)
    if rc != PA_OK:
        raise PaError(rc, "pa_calibrate_mfma")


def pa_calibrate_mfma_flops(num_workgroups: int, iters: int, fp8: bool = False) -> float:
    return float(lib().pa_calibrate_mfma_flops(int(num_workgroups), int(iters), int(bool(fp8))))
