"""GPU parity of logit soft-capping (softcap > 0) against the oracle, through
every entry point and every schedule: streamed and row-split prefill, the
key-split decode with and without split-KV, the mixed batch; bf16 and fp8
caches, causal and not; small batches element by element and the full-size
prefill and decode workloads on sampled rows."""
import numpy as np
import pytest

from paged_kv_gqa_attention_amd import synth
from tests import helpers as H
from tests.test_gpu_full import run_sampled
from tests.test_gpu_parity import run_and_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(10))
def test_softcap_prefill_and_mixed(seed):
    kv = "fp8_e4m3" if seed % 3 == 2 else "bf16"
    rng = np.random.default_rng(700 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    w = H.random_workload(700 + seed, kv_dtype=kv, causal=(seed % 4 != 3), max_len=300, G=G,
                          Hkv=int(rng.choice([1, 2])))
    w.softcap = float(rng.choice([0.5, 1.0, 2.0, 8.0]))   # scores ~N(0,1): the cap bends them
    ref = H.run_oracle(w)
    run_and_check(w, "prefill", ref=ref)
    run_and_check(w, "mixed", ref=ref)
    run_and_check(w, "mixed", num_splits=3, ref=ref)


@pytest.mark.parametrize("seed", range(8))
def test_softcap_decode(seed):
    kv = "fp8_e4m3" if seed % 2 else "bf16"
    rng = np.random.default_rng(800 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    w = H.random_workload(800 + seed, kv_dtype=kv, decode=True, max_len=900, G=G,
                          Hkv=int(rng.choice([1, 2, 3])), B=int(rng.integers(1, 9)))
    w.softcap = float(rng.choice([0.5, 1.0, 3.0]))
    ref = H.run_oracle(w)
    for s in (0, 1, 4):
        run_and_check(w, "decode", num_splits=s, ref=ref)
    run_and_check(w, "mixed", ref=ref)


@pytest.mark.slow
def test_softcap_full_size():
    w = synth.prefill_causal()
    w.softcap = 2.0
    run_sampled(w, "prefill", per_seq=3)
    w = synth.decode_llama8b()
    w.softcap = 1.0
    run_sampled(w, "decode")
    w = synth.decode_fp8_long()
    w.softcap = 1.5
    run_sampled(w, "decode", heads=8)
