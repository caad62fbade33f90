"""The calls the roofline figures are computed from, on the GPU: the device's compute
units and clock (the bf16 dense peak), one launch of the streaming-read calibration, and the
matrix-core rate calibration."""
import pytest
import torch

import gqa_attention_amd as g

pytestmark = pytest.mark.gpu


def test_device_info_names_the_device(gpu_available):
    info = g.device_info(0)
    assert info["compute_units"] > 0 and info["clock_khz"] > 0
    assert info["arch"].startswith("gfx950"), info
    assert info["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count


def test_stream_read_runs_and_leaves_the_sink(gpu_available):
    """Zero bytes fold to a zero checksum, which is not the launch's constant: the sink is
    not written, and the call leaves the buffer as it was."""
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((g.load_library().gqa_stream_read_sink_bytes(),), 7, dtype=torch.uint8,
                      device="cuda")
    for _ in range(3):
        g.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
    assert int(buf.count_nonzero()) == 0


def test_mfma_rate_sums_its_products(gpu_available):
    """Operands of bf16 ones: each product adds 16 to every element of its accumulator and
    each of a thread's 4 accumulators (16 elements) takes 4 products a round, so after 8
    rounds every thread's sum is 64 * 64 * 8 exactly; zeros give zero."""
    ones = torch.ones(1 << 16, dtype=torch.bfloat16, device="cuda")
    sink, flop = g.mfma_rate(ones, 8)
    torch.cuda.synchronize()
    assert flop == 256 * 8 * 8 * 16 * 2 * 32 * 32 * 16
    assert sink.numel() == 256 * 512
    assert bool((sink == 64 * 64 * 8).all())
    sink, _ = g.mfma_rate(torch.zeros_like(ones), 8, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
