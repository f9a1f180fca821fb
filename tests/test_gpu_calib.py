"""The MFMA-rate measurement kernel runs through the C ABI: on zero operands
every accumulator stays exactly zero, on random operands the sums are finite,
and the rate it implies is positive and below the published dense peak."""
import pytest
import torch

from paged_kv_gqa_attention_amd import binding

pytestmark = pytest.mark.gpu


def test_calibrate_mfma_runs_and_is_below_the_published_peak():
    nwg, iters = 64, 20
    ops = torch.randn(nwg * 32768, device="cuda").to(torch.bfloat16)
    sink = torch.full((nwg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    stream = binding.current_stream()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    ops.zero_()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream)
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    binding.pa_calibrate_mfma(ops, sink, nwg, iters, stream)
    e.record()
    torch.cuda.synchronize()
    tflops = binding.pa_calibrate_mfma_flops(nwg, iters) / (s.elapsed_time(e) * 1e-3) / 1e12
    assert 0 < tflops < 2516.6
