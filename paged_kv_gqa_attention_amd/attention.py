"""Thin torch-facing wrapper over the C ABI: device buffers, plan, workspace, runs.

Nothing here computes attention; it allocates outputs and the workspace with
torch and calls pa_run_prefill / pa_run_decode / pa_run_mixed of libpa.so.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


class DeviceInputs:
    """Device copies of a workload's tensors (q, pools, page table, lengths, descales)."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.device = torch.device(device)
        self.q = w.q.to(self.device)
        self.k_pool = w.k_pool.to(self.device)
        self.v_pool = w.v_pool.to(self.device)
        self.page_table = w.page_table.to(self.device)
        self.cu_q_lens = w.cu_q_lens.to(self.device)
        self.seq_lens = w.seq_lens.to(self.device)
        self.fp8 = w.kv_dtype == "fp8_e4m3"
        self.q_descale = (torch.tensor([w.q_descale], dtype=torch.float32, device=self.device)
                          if w.q_dtype == "fp8_e4m3" else None)
        if self.fp8:
            self.k_descale = torch.tensor([w.k_descale], dtype=torch.float32, device=self.device)
            self.v_descale = torch.tensor([w.v_descale], dtype=torch.float32, device=self.device)
        else:
            self.k_descale = self.v_descale = None


class PagedAttention:
    """A plan for one workload shape plus its workspace."""

    def __init__(self, w, *, num_splits: int = 0, num_cus: int = 0, device="cuda",
                 max_total_q: Optional[int] = None, max_seq_len: Optional[int] = None):
        self.w = w
        self.device = torch.device(device)
        kv = B.PA_KV_FP8_E4M3 if w.kv_dtype == "fp8_e4m3" else B.PA_KV_BF16
        self.desc = B.make_desc(
            num_seqs=w.num_seqs, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
            head_dim=w.head_dim, page_size=w.page_size, num_pages=w.num_pages,
            page_table_cols=w.pt_cols, page_table_row_stride=int(w.page_table.shape[1]),
            max_total_q=w.total_q if max_total_q is None else max_total_q,
            max_q_len=w.max_q_len,
            max_seq_len=w.max_seq_len if max_seq_len is None else max_seq_len,
            kv_dtype=kv, num_splits=num_splits, num_cus=num_cus,
            q_dtype=B.PA_Q_FP8_E4M3 if w.q_dtype == "fp8_e4m3" else B.PA_Q_BF16)
        self.plan = B.pa_plan(self.desc)
        self.info = B.pa_plan_get_info(self.plan)
        nbytes = B.pa_workspace_bytes(self.plan)
        self.workspace = (torch.empty(nbytes, dtype=torch.uint8, device=self.device)
                          if nbytes else None)
        if self.workspace is not None and self.workspace.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")

    def __del__(self):
        plan = getattr(self, "plan", None)
        if plan is not None:
            try:
                B.pa_plan_destroy(plan)
            except Exception:
                pass
            self.plan = None

    def args(self, x: DeviceInputs, out: torch.Tensor, lse: Optional[torch.Tensor],
             causal: Optional[bool] = None, scale: Optional[float] = None,
             workspace: Optional[torch.Tensor] = None, softcap: Optional[float] = None):
        return B.make_args(q=x.q, k_pool=x.k_pool, v_pool=x.v_pool, page_table=x.page_table,
                           cu_q_lens=x.cu_q_lens, seq_lens=x.seq_lens,
                           softmax_scale=self.w.scale if scale is None else scale,
                           causal=self.w.causal if causal is None else causal,
                           out=out, lse=lse, k_descale=x.k_descale, v_descale=x.v_descale,
                           workspace=self.workspace if workspace is None else workspace,
                           softcap=self.w.softcap if softcap is None else softcap,
                           q_descale=x.q_descale)

    def check(self, x: DeviceInputs) -> int:
        """Mask of metadata violations found on the device (0 = clean)."""
        flags = torch.full((1,), -1, dtype=torch.int32, device=self.device)
        a = self.args(x, None, None)                  # the check reads metadata only
        B.pa_check_metadata(self.plan, a, flags, B.current_stream())
        return int(flags.item())

    def new_outputs(self, x: DeviceInputs):
        T, Hq, D = x.q.shape                 # bf16 values or E4M3 codes: the same shape
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=self.device)
        lse = torch.empty((T, Hq), dtype=torch.float32, device=self.device)
        return out, lse

    def run(self, mode: str, x: DeviceInputs, out=None, lse=None, stream=None, **kw):
        """mode in {"prefill", "decode", "mixed"}; returns (out, lse)."""
        if out is None:
            out, lse = self.new_outputs(x)
        a = self.args(x, out, lse, **kw)
        s = B.current_stream() if stream is None else stream
        fn = {"prefill": B.pa_run_prefill, "decode": B.pa_run_decode,
              "mixed": B.pa_run_mixed}[mode]
        fn(self.plan, a, s)
        return out, lse


class MlaDecode:
    """An MLA decode plan for one latent-cache workload shape plus its workspace."""

    def __init__(self, w, *, num_splits: int = 0, num_cus: int = 0, device="cuda"):
        self.w = w
        self.device = torch.device(device)
        self.desc = B.pa_mla_desc(num_seqs=w.num_seqs, num_q_heads=w.num_q_heads,
                                  page_size=w.page_size, num_pages=w.num_pages,
                                  page_table_cols=w.pt_cols,
                                  page_table_row_stride=int(w.page_table.shape[1]),
                                  kv_page_stride=0, max_seq_len=w.max_seq_len,
                                  num_splits=num_splits, num_cus=num_cus)
        self.plan = B.pa_mla_plan(self.desc)
        self.num_splits = B.pa_mla_num_splits(self.plan)
        nbytes = B.pa_mla_workspace_bytes(self.plan)
        self.workspace = (torch.empty(nbytes, dtype=torch.uint8, device=self.device)
                          if nbytes else None)
        self.q = w.q.to(self.device)
        self.kv = w.kv.to(self.device)
        self.page_table = w.page_table.to(self.device)
        self.seq_lens = w.seq_lens.to(self.device)

    def __del__(self):
        plan = getattr(self, "plan", None)
        if plan is not None:
            try:
                B.pa_mla_plan_destroy(plan)
            except Exception:
                pass
            self.plan = None

    def new_outputs(self):
        out = torch.empty((self.w.num_seqs, self.w.num_q_heads, 512), dtype=torch.bfloat16,
                          device=self.device)
        lse = torch.empty((self.w.num_seqs, self.w.num_q_heads), dtype=torch.float32,
                          device=self.device)
        return out, lse

    def args(self, out, lse):
        return B.make_mla_args(q=self.q, kv_cache=self.kv, page_table=self.page_table,
                               seq_lens=self.seq_lens, softmax_scale=self.w.scale, out=out,
                               lse=lse, workspace=self.workspace, softcap=self.w.softcap)

    def run(self, out=None, lse=None, stream=None):
        if out is None:
            out, lse = self.new_outputs()
        B.pa_run_mla_decode(self.plan, self.args(out, lse),
                            B.current_stream() if stream is None else stream)
        return out, lse
