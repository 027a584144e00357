"""The streaming-read reference kernel reads every 16-byte element it is given (measurement
helper, not on the path): a lane writes the sink only when the XOR of the elements it read
equals the fixed key, so one element holding the key, in a buffer of zeros, must be seen."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz

from gpu_util import announce

pytestmark = pytest.mark.gpu

KEY = 0x9E3779B9   # the fixed key of kvz_stream_read


@pytest.mark.parametrize("n16,workgroups", [(1, 1), (4097, 3), (1 << 20, 0)])
def test_stream_read_sees_every_position(n16, workgroups):
    announce(f"stream read n16={n16} wg={workgroups}")
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvz.kvz_stream_read(buf, sink, workgroups)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0
    key = torch.tensor([np.int32(np.uint32(KEY).view(np.int32))], dtype=torch.int32, device="cuda")
    for j in sorted({0, n16 // 2, n16 - 1}):
        buf.zero_()
        buf[4 * j] = key[0]
        kvz.kvz_stream_read(buf, sink, workgroups)
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == KEY, f"element {j} not read"
        sink.zero_()
