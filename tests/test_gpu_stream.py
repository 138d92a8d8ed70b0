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


def test_prefetch_reads_every_range():
    """moe_prefetch over several ranges of ragged sizes: the XOR of its sink
    equals the XOR of every word of every range."""
    rng = np.random.default_rng(9)
    sizes = [16, 4096 * 3 + 32, (1 << 20) + 16 * 5, 5505024]
    bufs = [torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31 - 1, n // 4, dtype=np.int64).astype(np.int32)).cuda()
            for n in sizes]
    want = np.bitwise_xor.reduce(np.concatenate([b.cpu().numpy() for b in bufs]))
    for wg in (1, 33, 512):
        sink = torch.full((wg,), -1, dtype=torch.int32, device="cuda")
        say("prefetch ranges", len(bufs), "workgroups", wg)
        mb.prefetch(bufs, sink)
        torch.cuda.synchronize()
        assert np.bitwise_xor.reduce(sink.cpu().numpy()) == want


def test_block_unchanged_by_a_concurrent_prefetch():
    """A prefetch of the next block's router and shared-expert weights on a
    second stream, running while the block runs, leaves the block's output
    bits unchanged (it only reads)."""
    from tests import inputs
    from tests.test_gpu_parity import gpu_weights
    from tests.gpu_util import dev
    c = inputs.case("tp16_b1")
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = gpu_weights(c)
    X, Wr = dev(c.X), dev(c.Wr)
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    ref = torch.empty((cfg.B, cfg.d), dtype=torch.bfloat16, device="cuda")
    mb.moe_block(X, Wr, cfg.k, W13, W2, ref, ws, Ws13, Ws2)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    sink = torch.empty(64, dtype=torch.int32, device="cuda")
    for rep in range(3):
        out = torch.full_like(ref, float("nan"))
        ev = torch.cuda.Event()
        ev.record()
        side.wait_event(ev)
        mb.prefetch([Wr, Ws13, Ws2], sink, stream=side)
        mb.moe_block(X, Wr, cfg.k, W13, W2, out, ws, Ws13, Ws2)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
