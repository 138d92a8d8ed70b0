"""moe_block_noalloc, the allocation-free variant of moe_block (needs an
MI355X): called through the C ABI twice in a row, the second time with a
smaller batch, it gives the bits of moe_block on a workspace of its own --
ids, weights and output -- and meets the oracle's bars.  Its scratch keeps
the first call's contents when the second runs."""
import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from tests import inputs
from tests.gpu_util import check_block_output, dev, host, say
from tests.test_gpu_parity import gpu_weights

pytestmark = pytest.mark.gpu


def outputs(cfg):
    return (torch.full((cfg.B, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda"),
            torch.full((cfg.B, cfg.k), float("nan"), device="cuda"))


@pytest.mark.parametrize("first,second", [("tp8_b64", "tp16_b8"), ("tp16_b8", "tp16_b1")])
def test_noalloc_matches_moe_block_on_two_calls(first, second):
    for name in (first, second):
        c = inputs.case(name)
        cfg = c.cfg
        W13, W2, Ws13, Ws2 = gpu_weights(c)
        bias = None if c.bias is None else dev(c.bias)
        X, Wr = dev(c.X), dev(c.Wr)
        out_n, ids_n, w_n = outputs(cfg)
        mb.moe_block_noalloc(X, Wr, cfg.k, W13, W2, out_n, Ws13, Ws2, bias, c.bias_ld, ids_n, w_n)
        torch.cuda.synchronize()
        say("noalloc", name, mb.last_variant())
        out_w, ids_w, w_w = outputs(cfg)
        ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                             I=cfg.I, Is=cfg.Is))
        mb.moe_block(X, Wr, cfg.k, W13, W2, out_w, ws, Ws13, Ws2, bias, c.bias_ld, ids_w, w_w)
        torch.cuda.synchronize()
        assert torch.equal(ids_n, ids_w)
        assert torch.equal(w_n.view(torch.int32), w_w.view(torch.int32))
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
        assert np.array_equal(host(ids_n), c.ids)
        r_err, r_rnd = check_block_output(host(out_n), c.oracle_block()["out"])
        say("  max|err|/rms %.5f" % r_err)
        del W13, W2


def test_noalloc_rejects_before_launching():
    """Invalid arguments are refused on the host, before any launch."""
    A = 0x10000
    s = mb.lib.moe_block_noalloc(mb.DT_BF16, 65, 7168, 384, 8, 128, 128, A, A, None, 0, A, A, A, A, A,
                                 None, None, None)
    assert s == mb.EUNSUPPORTED
    s = mb.lib.moe_block_noalloc(mb.DT_BF16, 1, 7168, 384, 8, 128, 128, A, A, None, 0, A, A, A, A, A + 4,
                                 None, None, None)
    assert s == mb.EINVAL
