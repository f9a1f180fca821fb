"""GPU behaviour of pa_check_metadata: clean metadata reads 0 (poisoned dead
page-table columns included); each planted violation -- a live page id
outside the pool, a query run longer than its sequence, a sequence longer
than its page-table row, a decreasing cu_q_lens -- sets its bit and only it.
The check reads metadata only, so the planted values are never used as
addresses (no attention run is made on them)."""
import numpy as np
import pytest
import torch

from paged_kv_gqa_attention_amd import binding as B
from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H

pytestmark = pytest.mark.gpu


def fresh(seed=5):
    w = H.random_workload(seed, B=6, max_len=300, page=16)
    return w, DeviceInputs(w), PagedAttention(w)


def test_clean_metadata_reads_zero():
    for seed in range(6):
        w, x, pa = fresh(seed)
        assert pa.check(x) == 0, w.name
    w = synth.decode_llama8b()
    x = DeviceInputs(w)
    assert PagedAttention(w).check(x) == 0
    w = synth.mixed_24b(shuffle=True)
    x = DeviceInputs(w)
    assert PagedAttention(w).check(x) == 0


def test_planted_violations_set_their_bits():
    w, x, pa = fresh()
    L = w.seq_lens.numpy()
    b = int(np.argmax(L))
    live = (int(L[b]) + w.page_size - 1) // w.page_size
    # a dead column (past the live pages) may hold anything
    if live < w.pt_cols:
        x.page_table[b, live] = -5
        assert pa.check(x) == 0
    # a live column naming a page outside the pool
    keep = int(x.page_table[b, live - 1])
    x.page_table[b, live - 1] = w.num_pages
    assert pa.check(x) == B.PA_CHECK_PAGE_ID
    x.page_table[b, live - 1] = -1
    assert pa.check(x) == B.PA_CHECK_PAGE_ID
    x.page_table[b, live - 1] = keep
    assert pa.check(x) == 0
    # a sequence longer than its page-table row
    sl = x.seq_lens.clone()
    x.seq_lens[b] = w.pt_cols * w.page_size + 1
    assert pa.check(x) & B.PA_CHECK_SEQ_LEN
    x.seq_lens.copy_(sl)
    # a query run longer than its sequence: shrink a sequence under its q_len
    ql = np.diff(w.cu_q_lens.numpy())
    j = int(np.argmax(ql))
    if ql[j] > 1:
        x.seq_lens[j] = int(ql[j]) - 1
        assert pa.check(x) == B.PA_CHECK_Q_LEN
        x.seq_lens.copy_(sl)
    # cu_q_lens decreasing
    cu = x.cu_q_lens.clone()
    x.cu_q_lens[1] = x.cu_q_lens[2] + 1
    assert pa.check(x) & B.PA_CHECK_CU_Q_LENS
    x.cu_q_lens.copy_(cu)
    assert pa.check(x) == 0
