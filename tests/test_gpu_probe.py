"""kvq_read_probe: reads its buffer and leaves it, and (in practice) the sink,
as they were; the read rate it gives is reported by bench.py."""
import pytest
import torch

from _gpu_util import DEV, kq, need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 64 << 20])
def test_read_probe_reads_without_writing(nbytes):
    need_gpu()
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    before = buf.clone()
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    kq.kvq_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    # the probe stores only when the XOR of all it read is 0x9E3779B9
    assert int(sink.item()) in (7, 0x9E3779B9 - (1 << 32))
