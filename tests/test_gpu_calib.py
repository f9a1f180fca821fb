"""The MFMA-rate measurement kernel runs through the C ABI, for bf16 and E4M3
operands: on zero operands every accumulator stays exactly zero, on random
operands the sums are finite, and the rate it implies is positive and below
the published dense peak of its type."""
import pytest
import torch

from paged_kv_gqa_attention_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fp8", [False, True])
def test_calibrate_mfma_runs_and_is_below_the_published_peak(fp8):
    nwg, iters = 64, 20
    words = nwg * (65536 if fp8 else 32768)
    x = torch.randn(words * (2 if fp8 else 1), device="cuda")
    ops = x.to(torch.float8_e4m3fn).view(torch.int16) if fp8 else x.to(torch.bfloat16)
    sink = torch.full((nwg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    stream = binding.current_stream()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream, fp8=fp8)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    ops.zero_()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream, fp8=fp8)
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream, fp8=fp8)
    e.record()
    torch.cuda.synchronize()
    tflops = binding.pa_calibrate_mfma_flops(nwg, iters, fp8=fp8) / (s.elapsed_time(e) * 1e-3) / 1e12
    assert 0 < tflops < (5033.2 if fp8 else 2516.6)
