"""The Python binding's argument checks, on the host (no GPU): every tensor's
shape, dtype and contiguity, then its device, are checked before the C call,
because the C side gets only pointers and sizes.  Host tensors are built
here; every call below must raise before any pointer reaches the library."""
import pytest
import torch

from moe_block_skinny_amd import binding as mb

B, d, E, k, I, Is = 2, 64, 8, 2, 32, 32
bf = torch.bfloat16


def block_args(**over):
    a = dict(X=torch.zeros(B, d, dtype=bf), Wr=torch.zeros(E, d, dtype=bf), k=k,
             W13=torch.zeros(E, 2 * I, d, dtype=bf), W2=torch.zeros(E, d, I, dtype=bf),
             out=torch.zeros(B, d, dtype=bf), ws=torch.zeros(1024, dtype=torch.uint8),
             Ws13=torch.zeros(2 * Is, d, dtype=bf), Ws2=torch.zeros(d, Is, dtype=bf),
             bias=None, bias_ld=0, topk_ids=None, topk_w=None)
    a.update(over)
    return a


BAD_BLOCK = {
    "short router": (dict(Wr=torch.zeros(E - 1, d, dtype=bf)), ValueError),
    "W2 not [E][d][I]": (dict(W2=torch.zeros(E, I, d, dtype=bf)), ValueError),
    "W2 transposed view": (dict(W2=torch.zeros(E, I, d, dtype=bf).transpose(1, 2)), ValueError),
    "W13 odd rows": (dict(W13=torch.zeros(E, 2 * I + 1, d, dtype=bf)), ValueError),
    "W13 dtype": (dict(W13=torch.zeros(E, 2 * I, d, dtype=torch.float32)), TypeError),
    "out dtype": (dict(out=torch.zeros(B, d, dtype=torch.float32)), TypeError),
    "out shape": (dict(out=torch.zeros(B, d + 8, dtype=bf)), ValueError),
    "shared half given": (dict(Ws2=None), ValueError),
    "shared down shape": (dict(Ws2=torch.zeros(Is, d, dtype=bf)), ValueError),
    "bias per token with ld 0": (dict(bias=torch.zeros(B, E)), ValueError),
    "bias ld": (dict(bias=torch.zeros(E), bias_ld=3), ValueError),
    "bias dtype": (dict(bias=torch.zeros(E, dtype=bf)), TypeError),
    "ids shape": (dict(topk_ids=torch.zeros(B, k + 1, dtype=torch.int32)), ValueError),
    "ids dtype": (dict(topk_ids=torch.zeros(B, k, dtype=torch.int64)), TypeError),
    "weights dtype": (dict(topk_w=torch.zeros(B, k, dtype=bf)), TypeError),
    "X not a tensor": (dict(X=[[0.0] * d] * B), TypeError),
    "workspace dtype": (dict(ws=torch.zeros(256, dtype=torch.float32)), TypeError),
    "workspace strided": (dict(ws=torch.zeros(2048, dtype=torch.uint8)[::2]), ValueError),
}


@pytest.mark.parametrize("case", sorted(BAD_BLOCK))
def test_block_rejects(case):
    over, exc = BAD_BLOCK[case]
    with pytest.raises(exc):
        mb.moe_block(**block_args(**over))


def test_block_rejects_host_memory_last():
    """Well-formed arguments in host memory: the device check refuses them."""
    with pytest.raises(ValueError, match="GPU memory"):
        mb.moe_block(**block_args())


def test_dense_rejects():
    X, W = torch.zeros(4, 256, dtype=bf), torch.zeros(64, 256, dtype=bf)
    with pytest.raises(ValueError):
        mb.skinny_gemm(X, torch.zeros(64, 128, dtype=bf), torch.zeros(4, 64, dtype=bf))
    with pytest.raises(ValueError):
        mb.skinny_gemm(X, torch.zeros(256, 64, dtype=bf).t(), torch.zeros(4, 64, dtype=bf))
    with pytest.raises(TypeError):
        mb.skinny_gemm(X, W, torch.zeros(4, 64, dtype=torch.float16))
    with pytest.raises(ValueError):
        mb.skinny_gemm(X, W, torch.zeros(64, 4, dtype=bf))
    with pytest.raises(ValueError):
        mb.skinny_gemm_residual(X, W, torch.zeros(4, 32, dtype=bf), torch.zeros(4, 64, dtype=bf))
    with pytest.raises(ValueError):
        mb.skinny_gemm_residual(X, W, None, torch.zeros(4, 64, dtype=bf))
    with pytest.raises(ValueError, match="GPU memory"):
        mb.skinny_gemm(X, W, torch.zeros(4, 64, dtype=bf))


def test_route_ffn_combine_reject():
    X, Wr = torch.zeros(B, d, dtype=bf), torch.zeros(E, d, dtype=bf)
    ids, w = torch.zeros(B, k, dtype=torch.int32), torch.zeros(B, k)
    plan = torch.zeros(mb.plan_words(B, k, E), dtype=torch.int32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError):
        mb.moe_route(X, Wr, k, ids, w, plan[:-1], ws)
    with pytest.raises(ValueError):
        mb.moe_route(X, Wr, k, ids, w, plan, ws, logits_out=torch.zeros(B, E + 1))
    with pytest.raises(ValueError, match="GPU memory"):
        mb.moe_route(X, Wr, k, ids, w, plan, ws)
    W13, W2 = torch.zeros(E, 2 * I, d, dtype=bf), torch.zeros(E, d, I, dtype=bf)
    with pytest.raises(ValueError):
        mb.moe_expert_ffn(X, plan, W13, W2, k, torch.zeros(B, k, d), ws)
    with pytest.raises(ValueError):
        mb.moe_expert_ffn(X, plan, W13, torch.zeros(E - 1, d, I, dtype=bf), k, torch.zeros(B, k + 1, d), ws)
    with pytest.raises(ValueError):
        mb.moe_combine(torch.zeros(B, k + 1, d), torch.zeros(B, k + 1), True, torch.zeros(B, d, dtype=bf))
    with pytest.raises(ValueError, match="GPU memory"):
        mb.moe_combine(torch.zeros(B, k + 1, d), torch.zeros(B, k), True, torch.zeros(B, d, dtype=bf))
