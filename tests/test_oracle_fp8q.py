"""Pins of the oracle's fp8 queries (E4M3 codes times q_descale), CPU only.

Against torch's CPU flash-attention operator in float64 on queries decoded
with torch's float8_e4m3fn cast; and, for a power-of-two descale (where the
decoded queries are exact bf16 values), bit-identical to the bf16-query
oracle run on those values.  Planted mistakes are caught."""
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from tests import helpers as H

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")


def failures() -> int:
    bad = 0
    for seed, D in ((1, 64), (2, 128), (3, 128)):
        w = H.random_workload(500 + seed, kv_dtype="fp8_e4m3", D=D, q_dtype="fp8_e4m3",
                              causal=seed != 3, max_len=70)
        o, l = H.run_oracle(w)
        ro, rl = H.library_attention(w)
        bad += int(not (np.max(np.abs(o - ro)) < 1e-11 and np.max(np.abs(l - rl)) < 1e-11))
    return bad


def test_fp8_queries_match_library_attention():
    assert failures() == 0


def test_power_of_two_descale_equals_bf16_queries_bitwise():
    w = H.random_workload(510, kv_dtype="fp8_e4m3", D=128, q_dtype="fp8_e4m3", max_len=60)
    w.q_descale = 2.0 ** -5
    o8, l8 = H.run_oracle(w)
    qv = (w.q.view(torch.float8_e4m3fn).to(torch.float32) * w.q_descale).to(torch.bfloat16)
    assert torch.equal(qv.to(torch.float64), w.q.view(torch.float8_e4m3fn).to(torch.float64) * w.q_descale)
    wb = H.random_workload(510, kv_dtype="fp8_e4m3", D=128, max_len=60)
    wb.q = qv
    ob, lb = H.run_oracle(wb)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


MUTANTS = {
    "q_descale_dropped": ("pao_fp8_e4m3_to_double(((const uint8_t*)q)[t * q_stride + h * D + d]) * pr->q_descale",
                          "pao_fp8_e4m3_to_double(((const uint8_t*)q)[t * q_stride + h * D + d])"),
    "q_uses_k_descale": ("pao_fp8_e4m3_to_double(((const uint8_t*)q)[t * q_stride + h * D + d]) * pr->q_descale",
                         "pao_fp8_e4m3_to_double(((const uint8_t*)q)[t * q_stride + h * D + d]) * pr->k_descale"),
    "q_read_as_bf16": ("qrow[d] = pr->q_dtype == PAO_Q_FP8_E4M3", "qrow[d] = 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_fp8q_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, "mutation anchor not unique: " + name
    src = tmp_path / "pa_oracle.c"
    src.write_text(text.replace(before, after))
    shutil.copy(os.path.join(os.path.dirname(SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    assert failures() > 0, "planted mistake %s slipped through the fp8-query pins" % name
