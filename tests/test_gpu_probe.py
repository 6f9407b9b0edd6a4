"""GPU check of the measurement aid qd_stream_read (the practical HBM read
ceiling bench.py reports next to the 8 TB/s peak): it runs on buffers of
any multiple of 1 KiB, leaves the buffer untouched and reports no error."""
import pytest
import torch

import quantized_transformer_decode_amd as qd
from helpers import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1024, 37 * 1024, 1 << 20, 64 << 20])
def test_stream_read_runs_and_leaves_buffer(nbytes):
    print(f"stream_read bytes={nbytes}", flush=True)
    buf = torch.arange(nbytes, dtype=torch.int64, device=DEV).to(torch.uint8)
    before = buf.clone()
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    qd.stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_stream_read_rejects_bad_size():
    buf = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(qd.QDError) as e:
        qd.stream_read(buf, 1000, sink)
    assert e.value.status == qd.QD_ESHAPE
