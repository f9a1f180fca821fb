"""Benchmark: paged-KV GQA attention on one MI355X.

Headline line: the decode workload (B=256, Hq/Hkv 32/8, D 128, page 16,
seq_lens U[1024, 2048], bf16 K/V) through pa_run_decode, reported as KV GB/s
and as a fraction of the 8 TB/s HBM3E roof.  The other full-size workloads
(causal varlen prefill, unified mixed batch, fp8 long-context decode) and
the KV-cache append of the mixed batch's new tokens are timed too and
reported under "secondary".

The CPU leg (skipped with --no-cpu) is the only part that runs the fp64
oracle: it checks sampled rows of every timed attention workload against the
GPU output and times the oracle on a bounded sample of the headline workload
("cpu_baseline").  The append is checked without the oracle: every appended
element must equal the new row (bf16) or torch's own E4M3 cast of the
binary32 quotient (fp8), and nothing else in the pools may change.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-secondary] [--no-cpu]

One "step" is one call of the entry point over the whole batch (all kernels
of the call, the split-KV merge included), inputs already resident in HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn prefill TFLOP/s + decode KV GB/s, as % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
FP8_PEAK_TFLOPS = 2 * BF16_PEAK_TFLOPS
# fp8 queries on an fp8 cache: q.k and (on the tiles every row of a wave sees)
# p.v run on the E4M3 matrix cores, so the roof is the dense fp8 peak
FP8Q_PEAK_TFLOPS = FP8_PEAK_TFLOPS
KERNEL_SRC = os.path.join(ROOT, "paged_kv_gqa_attention_amd", "csrc", "pa_kernels.hip")
PROFILE_DIR = os.path.join(ROOT, "profiles")

O_TOL = {"bf16": 1.5e-2, "fp8_e4m3": 6e-2}
LSE_TOL = 1e-3


def kernel_sha() -> str:
    """Hash of the kernel source with comments and blank space removed, so
    that a recorded profile stays attached to the code it measured."""
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def read_profile(workload: str, kind: str, key: str):
    """A figure (`key: value`) from the committed rocprofv3 summary
    profiles/<workload>_<kind>.md, or None when absent or taken on a different
    kernel source."""
    path = os.path.join(PROFILE_DIR, "%s_%s.md" % (workload, kind))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sha:\s*([0-9a-f]+)", text)
    m_val = re.search(r"%s:\s*([0-9.eE+-]+)" % re.escape(key), text)
    if not m_sha or not m_val or m_sha.group(1) != kernel_sha():
        return None
    return float(m_val.group(1))


def read_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or None."""
    return read_profile(workload, "counters", "hbm_bytes_per_launch")


def read_counters(workload: str):
    """Measured HBM traffic and SQ figures of the workload's dominant kernel
    from the committed summaries (None where absent or stale)."""
    return {"traffic": read_traffic(workload),
            "mfma_busy_pct": read_profile(workload, "sq_counters", "mfma_busy_pct"),
            "lds_bank_conflicts_per_access": read_profile(workload, "sq_counters",
                                                          "lds_bank_conflicts_per_access")}


def validate(w, out, lse, rows, oracle_rows):
    o = out.float().cpu().numpy().reshape(-1, w.head_dim)[rows].astype(np.float64)
    l = lse.float().cpu().numpy().reshape(-1)[rows].astype(np.float64)
    ro, rl = oracle_rows
    eo = float(np.max(np.abs(o - ro)))
    el = float(np.max(np.abs(l - rl)))
    ok = bool(np.all(np.isfinite(o)) and eo <= O_TOL[w.kv_dtype] and el <= LSE_TOL)
    return ok, eo, el


def time_steps(fn, steps: int, warmup: int, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps       # ms per step


def bench_workload(name, mode, steps, warmup, cpu_leg, sample_rows_per_seq=2, heads=2,
                   softcap=0.0, num_splits=0, kv_dtype=None, q_dtype="bf16"):
    """Generate, time, and (CPU leg) check sampled rows.  Returns a result dict."""
    import torch
    from paged_kv_gqa_attention_amd import binding as B
    from paged_kv_gqa_attention_amd import synth
    from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention

    t0 = time.time()
    kw = {} if kv_dtype is None else {"kv_dtype": kv_dtype}
    if q_dtype != "bf16":
        kw["q_dtype"] = q_dtype
    w = synth.WORKLOADS[name](**kw)
    w.softcap = softcap
    gen_s = time.time() - t0
    x = DeviceInputs(w)
    pa = PagedAttention(w, num_splits=num_splits)
    out, lse = pa.new_outputs(x)
    stream = torch.cuda.current_stream()
    args = pa.args(x, out, lse)
    run = {"prefill": B.pa_run_prefill, "decode": B.pa_run_decode, "mixed": B.pa_run_mixed}[mode]
    s_ptr = int(stream.cuda_stream)

    def step():
        run(pa.plan, args, s_ptr)

    ms = time_steps(step, steps, warmup, stream)
    kv = w.kv_bytes()
    qo = w.qo_bytes()
    flops = w.flops()
    res = {
        "workload": name + ("_softcap%g" % softcap if softcap else "")
        + ("_fp8kv" if kv_dtype == "fp8_e4m3" and "fp8" not in name else "")
        + ("_fp8q" if q_dtype == "fp8_e4m3" else ""),
        "entry": "pa_run_" + mode, "ms_per_step": ms, "softcap": softcap,
        "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype,
        "kv_bytes": kv, "qo_bytes": qo, "flops": flops,
        "kv_gbs": kv / (ms * 1e-3) / 1e9,
        "alg_gbs": (kv + qo) / (ms * 1e-3) / 1e9,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "num_splits": int(pa.info.num_splits),
        "balanced_workgroups": int(pa.info.balanced_workgroups),
        "queue_workgroups": int(pa.info.queue_workgroups) if mode == "mixed" else 0,
        "validated_rows": 0, "max_abs_err_o": None, "max_abs_err_lse": None,
        "valid": None, "gen_s": round(gen_s, 2), "w": w,
    }
    if cpu_leg:
        rows = synth.sample_rows(w, per_seq=sample_rows_per_seq, heads=heads)
        ok, eo, el = oracle_check(w, out, lse, rows)
        res.update(validated_rows=len(rows), max_abs_err_o=eo, max_abs_err_lse=el, valid=ok)
    return res


def bench_append(kv_dtype, steps, warmup):
    """pa_run_append of the mixed batch's new tokens (8 chunks of 1000 plus 248
    decode tokens, Hkv 8, D 128, page 16).  Algorithmic bytes per launch: the
    new K and V rows read as bf16 plus the same elements written in the pool's
    dtype.  Checked by properties that hold at any size (no oracle)."""
    import torch
    from paged_kv_gqa_attention_amd import binding as B
    from paged_kv_gqa_attention_amd import synth
    from paged_kv_gqa_attention_amd.attention import DeviceInputs, PagedAttention

    w = synth.mixed_24b(kv_dtype=kv_dtype)
    x = DeviceInputs(w)
    pa = PagedAttention(w)
    T, Hkv, D = w.total_q, w.num_kv_heads, w.head_dim
    n = T * Hkv * D
    k_new = synth.normal_bf16(n, 11, 1).view(T, Hkv, D).cuda()
    v_new = synth.normal_bf16(n, 11, 2).view(T, Hkv, D).cuda()
    k_before, v_before = x.k_pool.clone(), x.v_pool.clone()
    a = B.make_append_args(k_new=k_new, v_new=v_new, cu_new=x.cu_q_lens, seq_lens=x.seq_lens,
                           page_table=x.page_table, k_pool=x.k_pool, v_pool=x.v_pool,
                           k_descale=x.k_descale, v_descale=x.v_descale)
    stream = torch.cuda.current_stream()
    s_ptr = int(stream.cuda_stream)

    def step():
        B.pa_run_append(pa.plan, a, s_ptr)

    ms = time_steps(step, steps, warmup, stream)
    # where every new token lands
    cu = w.cu_q_lens.numpy().astype(np.int64)
    L = w.seq_lens.numpy().astype(np.int64)
    seq = np.repeat(np.arange(w.num_seqs), np.diff(cu))
    pos = L[seq] - (cu[seq + 1] - cu[seq]) + (np.arange(T) - cu[seq])
    pages = torch.from_numpy(w.page_table.numpy()[seq, pos // w.page_size].astype(np.int64)).cuda()
    slots = torch.from_numpy((pos % w.page_size).astype(np.int64)).cuda()
    ok = True
    for new, pool, before, d in ((k_new, x.k_pool, k_before, w.k_descale),
                                 (v_new, x.v_pool, v_before, w.v_descale)):
        got = pool[pages, slots].cpu()
        if kv_dtype == "bf16":
            ok &= bool(torch.equal(got.view(torch.int16), new.cpu().view(torch.int16)))
        else:
            # the IEEE binary32 quotient (numpy divides exactly; torch on the GPU
            # multiplies by the divisor's reciprocal), then torch's RNE cast
            quot = new.cpu().float().numpy() / np.float32(d)
            want = torch.from_numpy(np.clip(quot, -448.0, 448.0)).to(torch.float8_e4m3fn)
            ok &= bool(torch.equal(got, want.view(torch.uint8)))
        rest = pool.clone()
        rest[pages, slots] = before[pages, slots]
        ok &= bool(torch.equal(rest.view(torch.uint8), before.view(torch.uint8)))
    esz = 2 if kv_dtype == "bf16" else 1
    alg = 2 * n * 2 + 2 * n * esz
    gbs = alg / (ms * 1e-3) / 1e9
    return {"workload": "append_mixed_24b_" + kv_dtype, "entry": "pa_run_append",
            "ms_per_step": ms, "new_tokens": T, "alg_bytes": alg, "alg_gbs": gbs,
            "bound": "hbm", "roofline_frac": gbs / HBM_PEAK_GBS, "valid": ok}


def bench_mla(name, steps, warmup, cpu_leg, num_splits=0):
    """pa_run_mla_decode over a latent-cache workload.  Algorithmic bytes: every
    live 576-wide bf16 row once, plus Q and O; flops 2 (576 + 512) per (query
    head, key)."""
    import torch
    from paged_kv_gqa_attention_amd import binding as B
    from paged_kv_gqa_attention_amd import synth
    from paged_kv_gqa_attention_amd.attention import MlaDecode

    w = synth.WORKLOADS[name]()
    m = MlaDecode(w, num_splits=num_splits)
    out, lse = m.new_outputs()
    a = m.args(out, lse)
    stream = torch.cuda.current_stream()
    s_ptr = int(stream.cuda_stream)

    def step():
        B.pa_run_mla_decode(m.plan, a, s_ptr)

    ms = time_steps(step, steps, warmup, stream)
    kv, qo, flops = w.kv_bytes(), w.qo_bytes(), w.flops()
    gbs = (kv + qo) / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": name, "entry": "pa_run_mla_decode", "ms_per_step": ms,
           "num_q_heads": w.num_q_heads, "num_splits": m.num_splits, "kv_bytes": kv,
           "qo_bytes": qo, "flops": flops, "alg_gbs": gbs, "tflops": tf, "bound": "hbm",
           "roofline_frac": max(gbs / HBM_PEAK_GBS, tf / BF16_PEAK_TFLOPS),
           "valid": None, "max_abs_err_o": None, "max_abs_err_lse": None}
    if cpu_leg:
        res.update(oracle_check_mla(w, out, lse))
    return res


# ---------------------------------------------------------------------------
# CPU leg: the only code here that runs the oracle
# ---------------------------------------------------------------------------

def oracle_check_mla(w, out, lse, n=96):
    """Sampled (sequence, head) rows of an MLA run against the fp64 oracle."""
    import torch
    import oracle
    rng = np.random.default_rng(5)
    rows = sorted(set(int(b) * w.num_q_heads + int(h) for b, h in
                      zip(rng.integers(0, w.num_seqs, n), rng.integers(0, w.num_q_heads, n))))
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    ro, rl = oracle.mla_decode(q_bits=bits(w.q), kv_cache=bits(w.kv),
                               page_table=w.page_table.numpy(), seq_lens=w.seq_lens.numpy(),
                               num_q_heads=w.num_q_heads, page_size=w.page_size, scale=w.scale,
                               rows=rows, pt_cols=w.pt_cols, softcap=w.softcap)
    o = out.float().cpu().numpy().reshape(-1, 512)[rows].astype(np.float64)
    l = lse.float().cpu().numpy().reshape(-1)[rows].astype(np.float64)
    eo = float(np.max(np.abs(o - ro)))
    el = float(np.max(np.abs(l - rl)))
    return {"valid": bool(np.all(np.isfinite(o)) and eo <= O_TOL["bf16"] and el <= LSE_TOL),
            "max_abs_err_o": eo, "max_abs_err_lse": el, "validated_rows": len(rows)}

def oracle_check(w, out, lse, rows):
    """Compare sampled output rows with the fp64 oracle's."""
    import oracle
    return validate(w, out, lse, rows, oracle.attention_workload(w, rows=rows))


def cpu_baseline(w, budget_s=10.0):
    """The oracle, untuned, on a bounded sample: groups of 16 whole sequences
    (all heads), in order and wrapping round, until about budget_s seconds of
    work; reports KV GB/s over the sample."""
    import oracle
    Hq = w.num_q_heads
    cu = w.cu_q_lens.numpy()
    L = w.seq_lens.numpy().astype(np.int64)
    threads = os.cpu_count() or 1
    done_bytes, elapsed, nseq = 0, 0.0, 0
    b = 0
    while elapsed < budget_s:
        take = min(w.num_seqs - b, 16)
        rows = np.arange(cu[b] * Hq, cu[b + take] * Hq, dtype=np.int64)
        t = time.time()
        oracle.attention_workload(w, rows=rows, threads=threads)
        elapsed += time.time() - t
        done_bytes += int(L[b:b + take].sum()) * w.num_kv_heads * w.head_dim * 2 * \
            (2 if w.kv_dtype == "bf16" else 1)
        nseq += take
        b = (b + take) % w.num_seqs
    return {"value": done_bytes / elapsed / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d sequence passes over the %d-sequence batch (all %d query heads), "
                      "%.1f s of fp64 CPU work" % (nseq, w.num_seqs, Hq, elapsed)}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def mfma_ceiling(iters: int = 1000, launches: int = 10):
    """Sustained dense MFMA rate of this GPU (pa_calibrate_mfma): two waves per
    SIMD doing nothing but v_mfma_f32_32x32x16_bf16, or E4M3
    v_mfma_scale_f32_32x32x64_f8f6f4, on random N(0,1) operands
    and, for comparison, on zeros (the chip's clock under a matrix-core load
    depends on how much the operand bits toggle).  The random-operand rates
    are the practical ceilings of the MFMA-bound lines; their roofline
    fractions stay taken against the published peaks."""
    import torch
    from paged_kv_gqa_attention_amd import binding
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device="cuda").manual_seed(7)
    stream = binding.current_stream()
    res = {}
    for fp8 in (False, True):
        # about 200 VGPRs per wave: two four-wave workgroups per compute unit,
        # every workgroup resident at once
        nwg = 2 * cus
        words = nwg * (65536 if fp8 else 32768)
        for kind in ("random", "zeros"):
            # E4M3: two codes per 16-bit word, every code a finite value
            x = torch.randn(words * (2 if fp8 else 1), generator=gen, device="cuda")
            if kind == "zeros":
                x.zero_()
            ops = x.to(torch.float8_e4m3fn).view(torch.int16) if fp8 else x.to(torch.bfloat16)
            sink = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")
            for _ in range(2):
                binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream, fp8=fp8)
            torch.cuda.synchronize()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(launches):
                binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream, fp8=fp8)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e) / launches
            res[(fp8, kind)] = binding.pa_calibrate_mfma_flops(nwg, iters, fp8=fp8) / (ms * 1e-3) / 1e12
    return {"tflops": round(res[(False, "random")], 1),
            "frac_of_peak": round(res[(False, "random")] / BF16_PEAK_TFLOPS, 4),
            "zero_operand_tflops": round(res[(False, "zeros")], 1),
            "fp8_tflops": round(res[(True, "random")], 1),
            "fp8_frac_of_peak": round(res[(True, "random")] / FP8_PEAK_TFLOPS, 4),
            "fp8_zero_operand_tflops": round(res[(True, "zeros")], 1),
            "kernel": "pa_calibrate_mfma: v_mfma_f32_32x32x16_bf16 only (8 accumulator chains), or "
                      "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3, no block scales; 4 chains) only, 2 waves per SIMD",
            "operands": "random N(0,1) bf16 / E4M3 (zero_operand_tflops: all zeros)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None, help="time one workload by name and print it")
    ap.add_argument("--softcap", type=float, default=0.0, help="logit soft cap for --only")
    ap.add_argument("--kv-dtype", default=None, choices=("bf16", "fp8_e4m3"),
                    help="cache dtype for --only (default: the workload's own)")
    ap.add_argument("--q-dtype", default="bf16", choices=("bf16", "fp8_e4m3"),
                    help="query dtype for --only (fp8_e4m3 needs an fp8 cache, prefill)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="plan num_splits for --only (0 heuristic, -1 balanced decode)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="measure the sustained bf16 MFMA rate on random operands and print it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy 5 times (HBM counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(got --gpus %d)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    modes = {"decode_llama8b": "decode", "prefill_causal": "prefill",
             "prefill_causal_d256": "prefill", "mixed_24b": "mixed", "decode_fp8_long": "decode"}

    def strip(r):
        return {k: v for k, v in r.items() if k != "w"}

    if a.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "repeats": 5}), flush=True)
        return
    if a.calibrate_mfma:
        print(json.dumps({"mfma_ceiling": mfma_ceiling()}), flush=True)
        return
    cpu_leg = not a.no_cpu
    if a.only:
        if a.only.startswith("append_"):
            r = bench_append(a.only[len("append_"):], a.steps, a.warmup)
        elif a.only.startswith("mla_"):
            r = bench_mla(a.only, a.steps, a.warmup, cpu_leg, num_splits=a.num_splits)
        else:
            r = bench_workload(a.only, modes[a.only], a.steps, a.warmup, cpu_leg,
                               softcap=a.softcap, num_splits=a.num_splits,
                               kv_dtype=a.kv_dtype, q_dtype=a.q_dtype)
        print(json.dumps(strip(r)), flush=True)
        return

    prim = bench_workload("decode_llama8b", "decode", a.steps, a.warmup, cpu_leg)
    print("# primary validated=%s err_o=%s err_lse=%s ms=%.4f" % (
        prim["valid"], prim["max_abs_err_o"], prim["max_abs_err_lse"], prim["ms_per_step"]),
        file=sys.stderr, flush=True)
    sec = {}
    if not a.no_secondary:
        for name in ("prefill_causal", "mixed_24b", "decode_fp8_long", "prefill_causal_d256"):
            # the prefills' CPU check covers 8 tokens x 8 heads of every sequence
            rp = (8, 8) if name.startswith("prefill") else (2, 2)
            r = bench_workload(name, modes[name], max(5, a.steps // 2), a.warmup, cpu_leg,
                               sample_rows_per_seq=rp[0], heads=rp[1])
            bound = "mfma" if name.startswith("prefill") else "hbm"
            if bound == "mfma":
                frac = r["tflops"] / BF16_PEAK_TFLOPS
            elif name == "mixed_24b":
                frac = max(r["tflops"] / BF16_PEAK_TFLOPS, r["alg_gbs"] / HBM_PEAK_GBS)
            else:
                frac = r["alg_gbs"] / HBM_PEAK_GBS
            e = strip(r)
            e["bound"] = bound
            e["roofline_frac"] = frac
            sec[name] = e
            print("# %s validated=%s ms=%.4f frac=%.3f" % (name, r["valid"], r["ms_per_step"], frac),
                  file=sys.stderr, flush=True)
        r = bench_workload("prefill_causal", "prefill", max(5, a.steps // 2), a.warmup, cpu_leg,
                           softcap=30.0)
        e = strip(r)
        e["bound"] = "mfma"
        e["roofline_frac"] = r["tflops"] / BF16_PEAK_TFLOPS
        sec[r["workload"]] = e
        print("# %s validated=%s ms=%.4f frac=%.3f" % (r["workload"], r["valid"], r["ms_per_step"],
                                                       e["roofline_frac"]),
              file=sys.stderr, flush=True)
        # fp8 cache, bf16 queries vs fp8 queries: the second runs its score
        # product and (off the diagonal) its PV product on the E4M3 matrix
        # cores, so it is measured against the dense fp8 peak (5.03 PFLOP/s)
        for qd in ("bf16", "fp8_e4m3"):
            r = bench_workload("prefill_causal", "prefill", max(5, a.steps // 2), a.warmup, cpu_leg,
                               kv_dtype="fp8_e4m3", q_dtype=qd)
            e = strip(r)
            e["bound"] = "mfma"
            e["peak_tflops"] = FP8Q_PEAK_TFLOPS if qd == "fp8_e4m3" else BF16_PEAK_TFLOPS
            e["roofline_frac"] = r["tflops"] / e["peak_tflops"]
            sec[r["workload"]] = e
            print("# %s validated=%s ms=%.4f frac=%.3f" % (r["workload"], r["valid"], r["ms_per_step"],
                                                           e["roofline_frac"]),
                  file=sys.stderr, flush=True)
        for name in ("mla_decode_h16", "mla_decode_h128"):
            r = bench_mla(name, a.steps, a.warmup, cpu_leg)
            sec[name] = r
            print("# %s validated=%s ms=%.4f frac=%.3f" % (name, r["valid"], r["ms_per_step"],
                                                           r["roofline_frac"]),
                  file=sys.stderr, flush=True)
        for kv in ("bf16", "fp8_e4m3"):
            r = bench_append(kv, a.steps, a.warmup)
            sec[r["workload"]] = r
            print("# %s validated=%s ms=%.4f frac=%.3f" % (r["workload"], r["valid"], r["ms_per_step"],
                                                           r["roofline_frac"]),
                  file=sys.stderr, flush=True)
    for name, e in sec.items():
        # the measured figures of each line's dominant kernel, beside its roofline
        if e["bound"] == "mfma" or (name.startswith(("mixed", "mla")) and
                                    e["tflops"] / BF16_PEAK_TFLOPS > e["alg_gbs"] / HBM_PEAK_GBS):
            peak = e.get("peak_tflops", BF16_PEAK_TFLOPS)
            roof = {"bound": "mfma", "achieved": round(e["tflops"], 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(e["tflops"] / peak, 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(e["alg_gbs"], 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(e["alg_gbs"] / HBM_PEAK_GBS, 4)}
        roof.update(read_counters(name))
        e["roofline"] = roof
    ceiling = mfma_ceiling() if sec else None
    if ceiling:
        for e in sec.values():
            if e["roofline"]["unit"] == "TFLOP/s" and e["roofline"]["peak"] == BF16_PEAK_TFLOPS:
                e["roofline"]["frac_of_mfma_ceiling"] = round(e["roofline"]["achieved"] / ceiling["tflops"], 4)
            elif e["roofline"]["unit"] == "TFLOP/s" and e["roofline"]["peak"] == FP8_PEAK_TFLOPS:
                e["roofline"]["frac_of_mfma_ceiling"] = round(e["roofline"]["achieved"] / ceiling["fp8_tflops"], 4)
    w = prim["w"]
    alg_bytes = prim["kv_bytes"] + prim["qo_bytes"]
    achieved = alg_bytes / (prim["ms_per_step"] * 1e-3) / 1e9
    cpu = None if a.no_cpu else cpu_baseline(w)
    line = {
        "metric": METRIC,
        "value": round(prim["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_llama8b", "entry": "pa_run_decode", "num_seqs": 256,
                   "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
                   "seq_lens": "U[1024,2048] seed 2", "kv_dtype": "bf16",
                   "num_splits": prim["num_splits"], "parallelism": "single GPU"},
        "valid": prim["valid"],
        "max_abs_err_o": prim["max_abs_err_o"],
        "max_abs_err_lse": prim["max_abs_err_lse"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("decode_llama8b"),
                     "mfma_busy_pct": read_profile("decode_llama8b", "sq_counters", "mfma_busy_pct"),
                     "kernel": "attn_kernel<128, bf16, decode>",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
        "secondary": sec,
        "mfma_ceiling": ceiling,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
