"""The two calls the roofline figures are computed from, on the GPU: the device's compute
units and clock (the bf16 dense peak), and one launch of the streaming-read calibration."""
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
