"""libpa.so without a GPU: every declared symbol is exported, plans validate
geometry and fail closed, workspace sizes follow the split choice, and runs
reject bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from paged_kv_gqa_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(B.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def desc(**kw):
    d = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
             num_pages=100, page_table_cols=16, max_total_q=4, max_q_len=1, max_seq_len=256,
             kv_dtype=B.PA_KV_BF16, num_splits=0, num_cus=256)
    d.update(kw)
    return B.make_desc(**d)


def plan_status(**kw):
    try:
        p = B.pa_plan(desc(**kw))
    except B.PaError as e:
        return e.code
    B.pa_plan_destroy(p)
    return B.PA_OK


def test_status_strings():
    for code in (B.PA_OK, B.PA_ERR_INVALID, B.PA_ERR_UNSUPPORTED, B.PA_ERR_WORKSPACE, B.PA_ERR_HIP,
                 B.PA_ERR_SCRATCH):
        assert B.pa_status_str(code).startswith("PA_")
    assert "unknown" in B.pa_status_str(-99)


def test_static_decode_host_checks():
    # the allocation-free decode refuses, before touching any device, a plan
    # whose scratch exceeds its static array, a NULL plan or arguments, and a
    # plan with more than one query token per sequence
    p = B.pa_plan(desc(num_seqs=4, num_q_heads=64, num_kv_heads=2, head_dim=256, page_size=128,
                       page_table_cols=64, max_total_q=4096, max_seq_len=8192,
                       kv_dtype=B.PA_KV_FP8_E4M3, num_splits=4))
    try:
        assert B.pa_workspace_bytes(p) > B.PA_STATIC_SCRATCH_BYTES
        a = B.pa_args()
        assert B.lib().pa_run_decode_static(p, ctypes.byref(a), None) == B.PA_ERR_SCRATCH
        assert B.lib().pa_run_decode_static(p, None, None) == B.PA_ERR_INVALID
        assert B.lib().pa_run_decode_static(None, ctypes.byref(a), None) == B.PA_ERR_INVALID
    finally:
        B.pa_plan_destroy(p)
    p = B.pa_plan(desc(max_q_len=2, max_total_q=8))
    try:
        a = B.pa_args()
        assert B.lib().pa_run_decode_static(p, ctypes.byref(a), None) == B.PA_ERR_INVALID
    finally:
        B.pa_plan_destroy(p)


@pytest.mark.parametrize("kw,code", [
    ({}, B.PA_OK),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(head_dim=512), B.PA_ERR_UNSUPPORTED),
    (dict(page_size=8), B.PA_ERR_UNSUPPORTED),
    (dict(page_size=256), B.PA_ERR_UNSUPPORTED),
    (dict(page_size=48), B.PA_ERR_UNSUPPORTED),
    (dict(num_q_heads=24, num_kv_heads=8), B.PA_ERR_UNSUPPORTED),     # G = 3
    (dict(num_q_heads=64, num_kv_heads=1), B.PA_ERR_UNSUPPORTED),     # G = 64 > 32
    (dict(num_q_heads=30, num_kv_heads=8), B.PA_ERR_INVALID),         # Hq % Hkv
    (dict(num_kv_heads=0), B.PA_ERR_INVALID),
    (dict(num_seqs=-1), B.PA_ERR_INVALID),
    (dict(page_table_cols=8, page_table_row_stride=4), B.PA_ERR_INVALID),
    (dict(kv_dtype=7), B.PA_ERR_INVALID),
    (dict(max_seq_len=10_000), B.PA_ERR_INVALID),                    # > C * page
    (dict(kv_page_stride=100), B.PA_ERR_INVALID),                     # < dense page
    (dict(kv_page_stride=1 << 31), B.PA_ERR_UNSUPPORTED),             # page bytes >= 2^32
    (dict(kv_page_stride=(1 << 31) - 8), B.PA_OK),                    # page bytes < 2^32
    (dict(num_q_heads=32768, num_kv_heads=32768, head_dim=256), B.PA_ERR_UNSUPPORTED),  # slot stride 2^24 bytes
    (dict(num_splits=-2), B.PA_ERR_INVALID),
    (dict(num_q_heads=64, num_kv_heads=2, head_dim=256, page_size=128, kv_dtype=B.PA_KV_FP8_E4M3), B.PA_OK),
    (dict(num_q_heads=4, num_kv_heads=4, head_dim=64), B.PA_OK),       # MHA
    (dict(num_seqs=0, max_total_q=0), B.PA_OK),                        # empty batch
    (dict(q_dtype=B.PA_Q_FP8_E4M3, kv_dtype=B.PA_KV_FP8_E4M3), B.PA_OK),
    (dict(q_dtype=B.PA_Q_FP8_E4M3, kv_dtype=B.PA_KV_FP8_E4M3, head_dim=64), B.PA_OK),
    (dict(q_dtype=B.PA_Q_FP8_E4M3), B.PA_ERR_UNSUPPORTED),              # fp8 queries need an fp8 cache
    (dict(q_dtype=B.PA_Q_FP8_E4M3, kv_dtype=B.PA_KV_FP8_E4M3, head_dim=256, page_size=128),
     B.PA_ERR_UNSUPPORTED),
    (dict(q_dtype=5), B.PA_ERR_INVALID),
])
def test_plan_validation(kw, code):
    assert plan_status(**kw) == code


def test_plan_null_arguments():
    h = ctypes.c_void_p()
    assert B.lib().pa_plan(None, ctypes.byref(h)) == B.PA_ERR_INVALID
    d = desc()
    assert B.lib().pa_plan(ctypes.byref(d), None) == B.PA_ERR_INVALID
    assert B.pa_workspace_bytes(None) == 0
    B.pa_plan_destroy(None)


def test_split_heuristic_and_workspace():
    # few (sequence, head) items and long contexts: split; workspace holds partials
    p = B.pa_plan(desc(num_seqs=64, num_q_heads=64, num_kv_heads=2, head_dim=256, page_size=128,
                       page_table_cols=256, max_total_q=64, max_seq_len=32768,
                       kv_dtype=B.PA_KV_FP8_E4M3))
    info = B.pa_plan_get_info(p)
    S = info.num_splits
    assert S > 1 and info.split_keys % 128 == 0 and S * info.split_keys >= 256 * 128
    rows = S * 64 * 64
    assert B.pa_workspace_bytes(p) >= rows * 256 * 4 + rows * 4
    assert info.workspace_bytes == B.pa_workspace_bytes(p)
    # where it splits, the heuristic also runs decode balanced: one workgroup per
    # resident slot (one per CU at fp8 D 256), two partial records of G rows each
    W = info.balanced_workgroups
    assert W == 256
    assert B.pa_workspace_bytes(p) >= 2 * W * 32 * (256 + 1) * 4 + (4 + 64 + 1) * 4
    B.pa_plan_destroy(p)
    # many items: no split, no balanced decode; mixed runs on the task queues,
    # whose workspace is all the plan needs
    p = B.pa_plan(desc(num_seqs=256, page_table_cols=128, max_total_q=256, max_seq_len=2048))
    info = B.pa_plan_get_info(p)
    assert info.num_splits == 1 and info.balanced_workgroups == 0 and info.queue_workgroups == 512
    assert B.pa_workspace_bytes(p) == ((10 + 1024 + 2 * 257) * 4 + 255) // 256 * 256
    B.pa_plan_destroy(p)
    # balanced decode on request; below -1 is invalid
    p = B.pa_plan(desc(num_seqs=256, page_table_cols=128, max_total_q=256, max_seq_len=2048,
                       num_splits=-1))
    info = B.pa_plan_get_info(p)
    assert info.balanced_workgroups == 2 * 256 and info.num_splits == 1
    assert B.pa_workspace_bytes(p) >= 2 * 512 * 4 * (128 + 1) * 4
    # -1 also puts mixed runs on the task queues: one workgroup per resident
    # slot of the mixed kernel (two per CU at D 128 bf16); the workspace holds
    # 10 counters (8 prefill-list shares, decode list, spare), 1024 arrival
    # counters and two offset lists of B + 1
    assert info.queue_workgroups == 2 * 256
    assert B.pa_workspace_bytes(p) >= (10 + 1024 + 2 * 257) * 4
    B.pa_plan_destroy(p)
    assert plan_status(num_splits=-2) == B.PA_ERR_INVALID
    p = B.pa_plan(desc(num_seqs=4096, page_table_cols=16, max_total_q=4096, num_splits=-1))
    assert B.pa_plan_get_info(p).queue_workgroups == 512
    assert B.pa_workspace_bytes(p) >= (10 + 1024 + 2 * 4097) * 4
    B.pa_plan_destroy(p)
    p = B.pa_plan(desc(num_splits=1))
    assert B.pa_plan_get_info(p).queue_workgroups == 0
    B.pa_plan_destroy(p)
    # forced splits are honoured (rounded to whole 128-key windows)
    p = B.pa_plan(desc(num_splits=3, page_table_cols=64, max_seq_len=1024))
    info = B.pa_plan_get_info(p)
    assert info.num_splits == 3 and info.split_keys == 384
    B.pa_plan_destroy(p)
    # the windows cover max_seq_len, not the page-table capacity (256 pages of
    # 16 keys here): every window holds live keys
    p = B.pa_plan(desc(num_splits=4, page_table_cols=256, max_seq_len=1024))
    info = B.pa_plan_get_info(p)
    assert info.num_splits == 4 and info.split_keys == 256
    B.pa_plan_destroy(p)
    p = B.pa_plan(desc(num_splits=4, page_table_cols=256, max_seq_len=0))   # 0: the capacity
    assert B.pa_plan_get_info(p).split_keys == 1024
    B.pa_plan_destroy(p)


def test_prefill_block_shape():
    for D, G in ((64, 2), (128, 4), (256, 32)):
        p = B.pa_plan(desc(head_dim=D, num_q_heads=8 * G, num_kv_heads=8))
        info = B.pa_plan_get_info(p)
        assert info.group == G and info.q_block_tokens >= 1 and info.mixed_q_block_tokens >= 1
        B.pa_plan_destroy(p)


def test_runs_reject_bad_arguments_without_touching_the_device():
    p = B.pa_plan(desc())
    a = B.pa_args()                       # all pointers NULL
    a.softmax_scale = 0.1
    for fn in (B.lib().pa_run_decode, B.lib().pa_run_prefill, B.lib().pa_run_mixed):
        assert fn(p, ctypes.byref(a), None) == B.PA_ERR_INVALID
    assert B.lib().pa_run_decode(p, None, None) == B.PA_ERR_INVALID
    assert B.lib().pa_run_decode(None, ctypes.byref(a), None) == B.PA_ERR_INVALID
    # misaligned pointers, bad scale, bad strides: fake non-null addresses are
    # never dereferenced because validation fails first
    good = dict(q=4096, k_pool=8192, v_pool=12288, page_table=16384, cu_q_lens=20480,
                seq_lens=24576, out=28672)
    def args(**kw):
        v = dict(good)
        v.update(kw)
        x = B.pa_args(**{k: v[k] for k in good})
        x.softmax_scale = kw.get("scale", 0.1)
        x.q_stride_t = kw.get("q_stride_t", 0)
        x.o_stride_t = kw.get("o_stride_t", 0)
        x.softcap = kw.get("softcap", 0.0)
        return x
    for bad in (args(q=4100), args(out=28674), args(scale=0.0), args(scale=-1.0),
                args(scale=float("nan")), args(q_stride_t=4000), args(o_stride_t=4100),
                args(softcap=-1.0), args(softcap=float("nan")), args(softcap=float("inf"))):
        assert B.lib().pa_run_decode(p, ctypes.byref(bad), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)
    # fp8 without descales
    p = B.pa_plan(desc(kv_dtype=B.PA_KV_FP8_E4M3))
    x = args()
    assert B.lib().pa_run_decode(p, ctypes.byref(x), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)
    # fp8 queries: prefill only, with a q descale and 16-byte query rows
    p = B.pa_plan(desc(kv_dtype=B.PA_KV_FP8_E4M3, q_dtype=B.PA_Q_FP8_E4M3))
    x = args()
    x.k_descale, x.v_descale = 32768, 32772
    for fn in (B.lib().pa_run_decode, B.lib().pa_run_mixed):
        assert fn(p, ctypes.byref(x), None) == B.PA_ERR_UNSUPPORTED
    assert B.lib().pa_run_prefill(p, ctypes.byref(x), None) == B.PA_ERR_INVALID   # no q descale
    x.q_descale = 32776
    x.q_stride_t = 32 * 128 + 8
    assert B.lib().pa_run_prefill(p, ctypes.byref(x), None) == B.PA_ERR_INVALID   # row not 16-byte
    B.pa_plan_destroy(p)
    # a task-queue plan: mixed runs need the workspace
    p = B.pa_plan(desc(num_splits=-1))
    assert B.lib().pa_run_mixed(p, ctypes.byref(args()), None) == B.PA_ERR_WORKSPACE
    B.pa_plan_destroy(p)
    # a split plan without workspace
    p = B.pa_plan(desc(num_splits=4, page_table_cols=64, max_seq_len=1024))
    x = args()
    assert B.lib().pa_run_decode(p, ctypes.byref(x), None) == B.PA_ERR_WORKSPACE
    x.workspace = 1 << 20
    x.workspace_bytes = 16
    assert B.lib().pa_run_decode(p, ctypes.byref(x), None) == B.PA_ERR_WORKSPACE
    # prefill needs no workspace but needs cu_q_lens
    y = args(cu_q_lens=None)
    y.cu_q_lens = None
    assert B.lib().pa_run_prefill(p, ctypes.byref(y), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)


def test_append_rejects_bad_arguments_without_touching_the_device():
    p = B.pa_plan(desc())
    assert B.lib().pa_run_append(p, None, None) == B.PA_ERR_INVALID
    assert B.lib().pa_run_append(None, ctypes.byref(B.pa_append_args()), None) == B.PA_ERR_INVALID
    assert B.lib().pa_run_append(p, ctypes.byref(B.pa_append_args()), None) == B.PA_ERR_INVALID
    good = dict(k_new=4096, v_new=8192, cu_new=12288, seq_lens=16384, page_table=20480,
                k_pool=24576, v_pool=28672)
    def args(**kw):
        v = dict(good)
        v.update(kw)
        x = B.pa_append_args(**v)
        return x
    for bad in (args(k_new=4098), args(v_pool=28680), args(seq_lens=None),
                args(new_stride_t=12), args(new_stride_t=1028)):
        assert B.lib().pa_run_append(p, ctypes.byref(bad), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)
    p = B.pa_plan(desc(kv_dtype=B.PA_KV_FP8_E4M3))
    assert B.lib().pa_run_append(p, ctypes.byref(args()), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)
    p = B.pa_plan(desc(num_seqs=0))                      # nothing to append: no launch
    assert B.lib().pa_run_append(p, ctypes.byref(B.pa_append_args()), None) == B.PA_OK
    B.pa_plan_destroy(p)


def test_mla_plan():
    def mdesc(**kw):
        d = dict(num_seqs=64, num_q_heads=16, page_size=32, num_pages=4000, page_table_cols=64,
                 page_table_row_stride=64, kv_page_stride=0, max_seq_len=2048, num_splits=0,
                 num_cus=256)
        d.update(kw)
        return B.pa_mla_desc(**d)
    # one round of workgroups: 64 sequences x 4 windows on 256 CUs
    p = B.pa_mla_plan(mdesc())
    assert B.pa_mla_num_splits(p) == 4
    assert B.pa_mla_workspace_bytes(p) >= 4 * 64 * 16 * (512 + 1) * 4
    B.pa_mla_plan_destroy(p)
    # 128 heads take two head groups: two windows fill the round
    p = B.pa_mla_plan(mdesc(num_q_heads=128))
    assert B.pa_mla_num_splits(p) == 2
    B.pa_mla_plan_destroy(p)
    # balanced on request: one workgroup per CU, two records of the group's rows each
    p = B.pa_mla_plan(mdesc(num_splits=-1, num_q_heads=100))
    assert B.pa_mla_num_splits(p) == -1
    assert B.pa_mla_workspace_bytes(p) >= 2 * 256 * 64 * (512 + 1) * 4 + (4 + 64 + 1) * 4
    B.pa_mla_plan_destroy(p)
    # many sequences: no split, no workspace
    p = B.pa_mla_plan(mdesc(num_seqs=512))
    assert B.pa_mla_num_splits(p) == 1 and B.pa_mla_workspace_bytes(p) == 0
    B.pa_mla_plan_destroy(p)
    for bad, code in ((dict(num_q_heads=129), B.PA_ERR_UNSUPPORTED), (dict(page_size=8), B.PA_ERR_UNSUPPORTED),
                      (dict(num_splits=-2), B.PA_ERR_INVALID),
                      (dict(num_q_heads=0), B.PA_ERR_INVALID), (dict(max_seq_len=5000), B.PA_ERR_INVALID),
                      (dict(kv_page_stride=100), B.PA_ERR_INVALID)):
        with pytest.raises(B.PaError) as e:
            B.pa_mla_plan(mdesc(**bad))
        assert e.value.code == code
    # runs reject bad arguments before touching the device
    p = B.pa_mla_plan(mdesc())
    assert B.lib().pa_run_mla_decode(p, None, None) == B.PA_ERR_INVALID
    a = B.pa_mla_args(q=4096, kv_cache=8192, page_table=12288, seq_lens=16384, out=20480,
                      softmax_scale=0.1)
    assert B.lib().pa_run_mla_decode(p, ctypes.byref(a), None) == B.PA_ERR_WORKSPACE
    for field, val in (("q", 4100), ("softmax_scale", -1.0), ("softcap", float("nan")),
                       ("q_stride_t", 12)):
        x = B.pa_mla_args(q=4096, kv_cache=8192, page_table=12288, seq_lens=16384, out=20480,
                          softmax_scale=0.1, workspace=1 << 20, workspace_bytes=1 << 30)
        setattr(x, field, val)
        assert B.lib().pa_run_mla_decode(p, ctypes.byref(x), None) == B.PA_ERR_INVALID
    B.pa_mla_plan_destroy(p)


def test_check_metadata_rejects_bad_arguments_without_touching_the_device():
    p = B.pa_plan(desc())
    a = B.pa_args()                       # page table and lengths NULL
    assert B.lib().pa_check_metadata(p, ctypes.byref(a), ctypes.c_void_p(4096), None) == B.PA_ERR_INVALID
    a.page_table, a.seq_lens = 8192, 12288
    assert B.lib().pa_check_metadata(p, ctypes.byref(a), None, None) == B.PA_ERR_INVALID
    assert B.lib().pa_check_metadata(None, ctypes.byref(a), ctypes.c_void_p(4096), None) == B.PA_ERR_INVALID
    assert B.lib().pa_check_metadata(p, None, ctypes.c_void_p(4096), None) == B.PA_ERR_INVALID
    B.pa_plan_destroy(p)


def test_calibrate_mfma_rejects_bad_arguments_on_the_host():
    lib = B.lib()
    big = 1 << 40
    assert lib.pa_calibrate_mfma(None, big, None, big, 1, 1, 0, None) == B.PA_ERR_INVALID
    assert lib.pa_calibrate_mfma(16, big, 16, big, 0, 1, 0, None) == B.PA_ERR_INVALID
    assert lib.pa_calibrate_mfma(16, big, 16, big, 1, 0, 0, None) == B.PA_ERR_INVALID
    assert lib.pa_calibrate_mfma(8, big, 16, big, 1, 1, 0, None) == B.PA_ERR_INVALID     # operands not 16-byte aligned
    assert lib.pa_calibrate_mfma(16, big, 16, big, 1, 1, 2, None) == B.PA_ERR_INVALID    # fp8 flag outside {0, 1}
    # buffers one element short of what two workgroups read and write
    assert lib.pa_calibrate_mfma(16, 2 * 32768 - 1, 16, big, 2, 1, 0, None) == B.PA_ERR_INVALID
    assert lib.pa_calibrate_mfma(16, 2 * 65536 - 1, 16, big, 2, 1, 1, None) == B.PA_ERR_INVALID
    assert lib.pa_calibrate_mfma(16, big, 16, 2 * 256 - 1, 2, 1, 0, None) == B.PA_ERR_INVALID
    # 4 waves x 64 MFMAs per trip x 2*32*32*K flop (K = 16 bf16, 64 E4M3)
    assert lib.pa_calibrate_mfma_flops(3, 5, 0) == 3 * 4 * 5 * 64 * 32768
    assert lib.pa_calibrate_mfma_flops(3, 5, 1) == 3 * 4 * 5 * 64 * 131072
