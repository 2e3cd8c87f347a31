"""attn_probe_clock on the device: one-wave workgroups (one per XCD) report
the shader-clock cycles and 100 MHz real-time ticks of a bounded spin."""
import pytest

import exact_attention_87_amd as ea

pytestmark = pytest.mark.gpu


def test_probe_clock_reads_each_xcd():
    import torch

    dev = torch.device("cuda:0")
    buf = torch.zeros(16, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    assert ea.attn_probe_clock(buf.data_ptr(), 8, 100000, stream.cuda_stream) == ea.ATTN_OK
    torch.cuda.synchronize()
    v = buf.cpu().tolist()
    for i in range(8):
        cycles, ticks = v[2 * i], v[2 * i + 1]
        # the spin ends at the first real-time read past its 1 ms window
        assert 100000 <= ticks < 200000, (i, ticks)
        assert 300.0 < cycles / ticks * 100.0 < 3000.0, (i, cycles, ticks)


def test_probe_clock_beside_other_work():
    """A probe on a second stream finishes while a long kernel runs on the first."""
    import torch

    dev = torch.device("cuda:0")
    buf = torch.zeros(16, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(dev)
    a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    b = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert ea.attn_probe_clock(buf.data_ptr(), 8, 20000, side.cuda_stream) == ea.ATTN_OK
    for _ in range(20):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    v = buf.cpu().tolist()
    assert all(20000 <= v[2 * i + 1] for i in range(8))
    assert all(300.0 < v[2 * i] / v[2 * i + 1] * 100.0 < 3000.0 for i in range(8))


def test_probe_clock_long_window_is_not_cut_short():
    """A 0.4 s window runs to its end at the idle 2.4 GHz clock (the spin's
    iteration cap lies beyond the 2 s maximum)."""
    import torch

    dev = torch.device("cuda:0")
    buf = torch.zeros(2, dtype=torch.int64, device=dev)
    assert ea.attn_probe_clock(buf.data_ptr(), 1, 40_000_000,
                               torch.cuda.current_stream(dev).cuda_stream) == ea.ATTN_OK
    torch.cuda.synchronize()
    cycles, ticks = buf.cpu().tolist()
    assert 40_000_000 <= ticks < 40_100_000, ticks
    assert 300.0 < cycles / ticks * 100.0 < 3000.0
