"""GPU checks of the read-ceiling measurement (bitnest_stream_read) through
the C ABI: it must read every byte of the buffer it is given, exactly once
per lane fold, and nothing past it.

A buffer of zeros with one planted dword V: the lane that reads that 16-byte
slot folds to V, every other lane to 0, so sink[0] becomes V exactly when
the call is told that V is the value to report and the planted slot was
read; a slot that was skipped (or read twice: V xor V = 0) leaves the sink
untouched.
"""
import pytest
import torch

import w8_quantized_linear_amd as bn

pytestmark = pytest.mark.gpu

V = 0x13572468


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _sink():
    return torch.full((1,), -1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("kib", [1, 7, 2048 * 8 + 3, 8 * 1024, 12 * 1024 + 1])
@pytest.mark.parametrize("depth,wpc", [(2, 0), (4, 0), (8, 0), (4, 8), (8, 16)])
def test_every_sampled_slot_is_read_once(kib, depth, wpc):
    buf = torch.zeros(kib * 1024 // 4, dtype=torch.int32, device="cuda")
    n_dw = buf.numel()
    for pos in sorted({0, 5, n_dw // 2 + 1, n_dw - 4, n_dw - 1}):
        buf.zero_()
        buf[pos] = V
        s = _sink()
        bn.bitnest_stream_read(buf, s, never=V, depth=depth, waves_per_cu=wpc)
        torch.cuda.synchronize()
        assert s.item() == V, (kib, pos)
        # the same call told to report another value leaves the sink alone
        s = _sink()
        bn.bitnest_stream_read(buf, s, never=V ^ 1, depth=depth, waves_per_cu=wpc)
        torch.cuda.synchronize()
        assert s.item() == -1, (kib, pos)


@pytest.mark.parametrize("depth", [2, 4, 8])
def test_nothing_past_the_buffer_is_read(depth):
    # a planted value right after the given length must not be seen
    big = torch.zeros(4096 // 4 * 3, dtype=torch.int32, device="cuda")
    big[4096 // 4 * 2] = V
    s = _sink()
    bn.bitnest_stream_read(big[:4096 // 4 * 2], s, never=V, depth=depth)
    torch.cuda.synchronize()
    assert s.item() == -1
