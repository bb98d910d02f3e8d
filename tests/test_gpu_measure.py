"""The read-ceiling kernel bench.py reports beside every weight-streaming
figure: it must read the whole buffer (a sink write happens only for one
impossible accumulator value) and leave every other byte alone."""
import pytest
import torch

from gemm_rwkv_amd import rq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 33 * (1 << 20) + 16 * 7])
def test_stream_read_touches_nothing(nbytes):
    buf = torch.arange(nbytes, dtype=torch.int32, device="cuda").to(torch.uint8)
    ref = buf.clone()
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    rq.rq_stream_read(buf, nbytes, sink)
    rq.rq_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
    assert sink.tolist() == [7, 7, 7, 7]


def test_stream_read_zero_bytes():
    buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    rq.rq_stream_read(buf, 0, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0, 0, 0]
