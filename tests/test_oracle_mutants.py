"""The oracle's pins have teeth: plausible single mistakes planted in a copy of
the oracle's C source (CPU only) are each caught by the library-attention pin
or the fp8 codec pin."""
import os
import shutil

import numpy as np
import pytest
import torch

import oracle
from tests import helpers as H

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTANTS = {
    "causal_off_by_one": ("if (pr->causal && pos + 1 < hi) hi = pos + 1;",
                          "if (pr->causal && pos + 2 < hi) hi = pos + 2;"),
    "top_left_causal": ("const int64_t pos = L - q_len + i;", "const int64_t pos = i;"),
    "head_map_modulo": ("const int64_t g = h / G;", "const int64_t g = h % pr->num_kv_heads;"),
    "lse_sign": ("l += exp(s[j - lo] - m);\n  const double lse = m + log(l);",
                 "l += exp(s[j - lo] - m);\n  const double lse = m - log(l);"),
    "scale_dropped": ("s[j - lo] = pr->scale * dot;", "s[j - lo] = dot;"),
    "slot_shift": ("const int64_t slot = j % pr->page_size;\n    double dot",
                   "const int64_t slot = (j + 1) % pr->page_size;\n    double dot"),
    "kv_head_slot_swapped": ("const int64_t idx = page * page_stride + (slot * H + g) * D + d;",
                             "const int64_t idx = page * page_stride + (g * pr->page_size + slot) * D + d;"),
    "fp8_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                 "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_subnormal": ("mag = ldexp((double)m / 8.0, 1 - 7);", "mag = ldexp((double)m / 8.0, -7);"),
    "v_uses_k_descale": ("o_row[d] += p * kv_elem(pr, v_pool, phys, slot, g, d, pr->v_descale);",
                         "o_row[d] += p * kv_elem(pr, v_pool, phys, slot, g, d, pr->k_descale);"),
    "row_stride_ignored": ("page_table[b * pr->pt_row_stride + j / pr->page_size];\n    const int64_t slot = j % pr->page_size;\n    double",
                           "page_table[b * pr->pt_cols + j / pr->page_size];\n    const int64_t slot = j % pr->page_size;\n    double"),
}


def _caught(workloads) -> bool:
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got, want = oracle.fp8_e4m3_to_double(c), float(ref[c])
        if not (got == want or (np.isnan(got) and np.isnan(want))):
            return True
    for w in workloads:
        o, lse = H.run_oracle(w)
        ro, rl = H.library_attention(w)
        if not (np.max(np.abs(o - ro)) < 1e-11 and np.max(np.abs(lse - rl)) < 1e-11):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, "mutation anchor not unique: " + name
    src = tmp_path / "pa_oracle.c"
    src.write_text(text.replace(before, after))
    shutil.copy(os.path.join(os.path.dirname(SRC), "pa_oracle.h"), tmp_path / "pa_oracle.h")
    so = oracle.compile_source(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    ws = [H.random_workload(s, kv_dtype=kv, causal=True)
          for s, kv in ((1, "bf16"), (2, "fp8_e4m3"), (5, "bf16"))]
    # a workload whose page table has a wider row stride than its width
    from paged_kv_gqa_attention_amd import synth
    ws.append(synth.build(name="stride", seq_lens=[40, 70], q_lens=[40, 3], num_q_heads=4,
                          num_kv_heads=2, head_dim=64, page_size=16, seed=9, pt_cols=5,
                          pt_row_stride=11, threads=1))
    assert _caught(ws), "planted mistake %s slipped through every pin" % name


def test_unmutated_source_passes_the_same_checks(tmp_path, monkeypatch):
    so = oracle.compile_source(SRC, str(tmp_path / "libclean.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(so))
    ws = [H.random_workload(s, kv_dtype=kv, causal=True)
          for s, kv in ((1, "bf16"), (2, "fp8_e4m3"), (5, "bf16"))]
    assert not _caught(ws)
