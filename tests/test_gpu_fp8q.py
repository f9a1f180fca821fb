"""GPU parity of fp8 queries (E4M3 codes with a per-tensor descale) on an fp8
cache: the streamed prefill runs its score product on the E4M3 matrix cores.
The oracle takes the same codes times the same descales, so the comparison is
element by element at the fp8-cache tolerance (6e-2 on O, 1e-3 on LSE);
small random batches (head dim 64 and 128, causal or not, chunked rows, with
and without soft-capping) in full, and the full-size causal prefill on
sampled rows."""
import numpy as np
import pytest

from paged_kv_gqa_attention_amd import synth
from tests import helpers as H
from tests.test_gpu_full import run_sampled
from tests.test_gpu_parity import run_and_check

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


@pytest.mark.slow
def test_fp8_query_prefill_full_size():
    w = synth.prefill_causal(kv_dtype="fp8_e4m3", q_dtype="fp8_e4m3")
    run_sampled(w, "prefill", per_seq=6)
