"""The reference streams (bandwidth ceilings) on the GPU: they compute what they
say, over ragged sizes, so the bandwidth they report is for real work."""
from __future__ import annotations

import pytest
import torch

from _parity import DEV, announce

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cross_entropy_tv_amd as lx  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (64 << 20) + 32 * 1024 + 16])
def test_read2_write_is_the_xor_and_stops_at_the_end(nbytes):
    announce(f"reference streams, {nbytes} bytes")
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    n = nbytes // 4
    a = torch.randint(-2**31, 2**31 - 1, (n,), generator=g, device=DEV, dtype=torch.int32)
    b = torch.randint(-2**31, 2**31 - 1, (n,), generator=g, device=DEV, dtype=torch.int32)
    out = torch.full((n + 64,), 7, dtype=torch.int32, device=DEV)
    lx.lx_stream_read2_write(a, b, out[:n])
    torch.cuda.synchronize()
    assert torch.equal(out[:n], a ^ b)
    assert torch.all(out[n:] == 7), "wrote past the end"
    sink = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    lx.lx_stream_read(a, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) in (5, 0x9e3779b9 - 2**32)
