"""GPU parity of fp8 queries (E4M3 codes with a per-tensor descale) on an fp8
cache: the streamed prefill runs its score product on the E4M3 matrix cores,
and, for the 64-key tiles every row of a wave sees (rows with at least 256
keys), its PV product too, on probabilities quantised to E4M3.  The oracle
takes the same query and cache codes times the same descales and computes
the exact softmax (no probability quantisation), so the comparison is
element by element at the fp8-cache tolerance (6e-2 on O, 1e-3 on LSE):
small random batches (head dim 64 and 128, causal or not, chunked rows, with
and without soft-capping) in full, rows with few keys, and the full-size
causal prefill on rows covering every work item."""
import numpy as np
import pytest

import torch

from paged_kv_gqa_attention_amd import synth
from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention
from tests import helpers as H
from tests.test_gpu_parity import check, run_and_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(12))
def test_fp8_query_prefill(seed):
    rng = np.random.default_rng(900 + seed)
    w = H.random_workload(900 + seed, kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3",
                          D=int(rng.choice([64, 128])), causal=(seed % 4 != 3),
                          max_len=400, G=int(rng.choice([1, 2, 4, 8, 16, 32])),
                          Hkv=int(rng.choice([1, 2])))
    if seed % 3 == 1:
        w.softcap = float(rng.choice([1.0, 4.0]))
    run_and_check(w, "prefill")


def test_fp8_query_decode_rows_in_prefill():
    # q_len 1 rows and empty keys-only sequences through the streamed kernel
    w = synth.build(name="fp8q_dec", seq_lens=[1, 70, 129, 300], q_lens=[1, 1, 5, 300],
                    num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=16, seed=17,
                    kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3", threads=1)
    run_and_check(w, "prefill")


def test_fp8_query_long_rows_use_the_fp8_pv_product():
    # non-causal rows over 300-1,100 keys: every 64-key tile below the live
    # length goes through the E4M3 PV product
    w = synth.build(name="fp8q_long", seq_lens=[1100, 300, 640], q_lens=[40, 300, 7],
                    num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, seed=19,
                    kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3", causal=False, threads=1)
    run_and_check(w, "prefill")


@pytest.mark.slow
def test_fp8_query_prefill_full_size():
    w = synth.prefill_causal(kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3")
    pa = PagedAttention(w)
    rows = H.cover_rows(w, pa.info.q_block_tokens)
    print("case", w.name, "rows", len(rows), flush=True)
    x = DeviceInputs(w)
    out, lse = pa.run("prefill", x)
    torch.cuda.synchronize()
    ref = H.run_oracle(w, rows=rows)
    check(w, out, lse, ref[0], ref[1], rows=rows, what=w.name + "/fp8q/cover")
