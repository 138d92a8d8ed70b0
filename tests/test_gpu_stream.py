"""The read-only streaming yardstick (moe_stream_read) reads every word of
its buffer (needs an MI355X): the XOR of the per-workgroup results equals
the XOR of the buffer, for sizes that leave ragged slices and tails and for
grids from one workgroup to more slices than 4 KB steps."""
import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (3 << 20) + 16 * 7, 44040192])
@pytest.mark.parametrize("wg", [1, 7, 256, 2048])
def test_stream_read_reads_every_word(nbytes, wg):
    rng = np.random.default_rng(nbytes % 1000 + wg)
    host = rng.integers(-2 ** 31, 2 ** 31 - 1, nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.full((wg,), -1, dtype=torch.int32, device="cuda")
    say("stream_read bytes", nbytes, "workgroups", wg)
    mb.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)
