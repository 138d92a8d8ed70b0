"""The block at the edges of its scope, against the CPU oracle (needs an
MI355X): the largest routing problem the ABI accepts (B = 64 tokens, E = 512
experts, top-16: 1024 slots), every expert chosen by every token (k = E),
top-1, and the smallest batch that takes the matrix shapes (B = 9).  Expert
ids and the plan bit-exact; the block output within the bf16-aware bar of
check_block_output: per element |err| <= |bf16(ref) - ref| + 2e-3 rms, and
the stated max|err| <= 2e-2 rms wherever rounding the exact result to bf16
leaves room for it.  In the max-scope case it does not: its outputs reach
6.2 times their rms, and the exact result rounded to bf16 is already
0.0225 rms away from itself (asserted below), above the stated bar."""
import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from moe_block_skinny_amd import synth
from tests import inputs
from tests.gpu_util import check_block_output, dev, host, rms, say

pytestmark = pytest.mark.gpu

LIMITS = {
    "max_scope": synth.MoEConfig("max_scope", 64, 1024, 512, 16, 32, 32, "bf16", "plain"),
    "all_experts": synth.MoEConfig("all_experts", 5, 1024, 8, 8, 64, 0, "bf16", "plain"),
    "top1": synth.MoEConfig("top1", 64, 1024, 64, 1, 64, 64, "bf16", "zipf"),
    "first_matrix_b9": synth.MoEConfig("first_matrix_b9", 9, 2048, 32, 4, 64, 64, "bf16", "gumbel"),
}


def weights(c):
    cfg = c.cfg
    W13 = torch.full((cfg.E, 2 * cfg.I, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    W2 = torch.full((cfg.E, cfg.d, cfg.I), float("nan"), dtype=torch.bfloat16, device="cuda")
    for e in c.touched:
        W13[e] = dev(c.W13[e])
        W2[e] = dev(c.W2[e])
    Ws13 = None if c.Ws13 is None else dev(c.Ws13)
    Ws2 = None if c.Ws2 is None else dev(c.Ws2)
    return W13, W2, Ws13, Ws2


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_block_and_route_at_scope_limits(name):
    c = inputs.Case(LIMITS[name], seed=7)
    cfg = c.cfg
    say("limits", name, "distinct experts", len(c.touched), "redraws", c.redraws)
    W13, W2, Ws13, Ws2 = weights(c)
    bias = None if c.bias is None else dev(c.bias)
    X, Wr = dev(c.X), dev(c.Wr)
    # the block
    out = torch.full((cfg.B, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    mb.moe_block(X, Wr, cfg.k, W13, W2, out, ws, Ws13, Ws2, bias, c.bias_ld, ids, w)
    torch.cuda.synchronize()
    say("  variant", mb.last_variant())
    ref = c.oracle_block()["out"]
    g = host(out)
    assert np.array_equal(host(ids), c.ids)
    assert np.max(np.abs(host(w) - c.w)) <= 1e-5
    r_err, r_rnd = check_block_output(g, ref)
    say("  max|err|/rms %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
    if name == "max_scope":
        # rounding alone exceeds the stated bar here (outputs up to ~6.2 rms)
        assert 0.0220 <= r_rnd <= 0.0230
    # the router alone: ids, weights and the plan it builds itself
    rids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    rw = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    plan = torch.full((mb.plan_words(cfg.B, cfg.k, cfg.E),), -7, dtype=torch.int32, device="cuda")
    wsr = mb.workspace(mb.workspace_bytes(mb.OP_ROUTE, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k))
    mb.moe_route(X, Wr, cfg.k, rids, rw, plan, wsr, bias=bias, bias_ld=c.bias_ld)
    torch.cuda.synchronize()
    assert np.array_equal(host(rids), c.ids)
    assert np.array_equal(host(plan), c.plan)
    assert np.max(np.abs(host(rw) - c.w)) <= 1e-5


# The matrix-shape down at its edges: 17..32 rows per workgroup with the last
# workgroup's range cut short (d = 4128: 20 rows per workgroup, 8 in the
# last; d = 5120: 20 rows, a 4-row second half), a shared expert with another
# intermediate size than the routed ones (its h tiles are read with the
# wider row stride), no shared expert, and the matrix shape forced at a
# batch that would take the vector shape (entries of one to a few tokens,
# h tiles mostly padding).
EDGES = {
    "rows20_shared_wider": (synth.MoEConfig("rows20_shared_wider", 24, 5120, 64, 4, 64, 96, "bf16", "gumbel"), None),
    "ragged_tail_no_shared": (synth.MoEConfig("ragged_tail_no_shared", 64, 4128, 32, 2, 128, 0, "bf16", "zipf"), None),
    "forced_matrix_b4": (synth.MoEConfig("forced_matrix_b4", 4, 7168, 64, 8, 128, 128, "bf16", "gumbel"), "mfma"),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_block_matrix_down_edges(name):
    cfg0, force = EDGES[name]
    c = inputs.Case(cfg0, seed=11)
    cfg = c.cfg
    say("matrix down edge", name, "distinct experts", len(c.touched))
    W13, W2, Ws13, Ws2 = weights(c)
    bias = None if c.bias is None else dev(c.bias)
    out = torch.full((cfg.B, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    prev = mb.set_variant(force) if force else None
    try:
        mb.moe_block(dev(c.X), dev(c.Wr), cfg.k, W13, W2, out, ws, Ws13, Ws2, bias, c.bias_ld, ids, w)
        torch.cuda.synchronize()
        say("  variant", mb.last_variant())
    finally:
        if force:
            mb.set_variant(prev)
    ref = c.oracle_block()["out"]
    g = host(out)
    assert np.array_equal(host(ids), c.ids)
    assert np.max(np.abs(host(w) - c.w)) <= 1e-5
    r_err, r_rnd = check_block_output(g, ref)
    say("  max|err|/rms %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
    assert r_rnd + 2e-3 <= 2e-2    # the stated bar applies here and was asserted


def test_block_gate_up_cuts_heaviest_entries_first():
    """Batch 64 (Zipf routing) with a routing where cutting every entry of
    more than 16 tokens into two K halves would need more gate/up tasks than
    the launch has workgroups (512), but cutting those of more than 32 fits:
    the cut then covers only the heavier entries.  The case is checked to be
    one (counted from the oracle's routing), then the block against the
    oracle as above."""
    cfg = synth.CONFIGS["tp8_b64"]
    c = inputs.Case(cfg, seed=1)
    _, cnt = np.unique(c.ids, return_counts=True)
    ms = list(cnt) + [cfg.B]                 # routed entries, then the shared one
    tiles = 2 * cfg.I // 64                  # 64-row tasks per entry
    t1 = tiles * len(ms)
    assert t1 + tiles * sum(m > 16 for m in ms) > 512
    assert t1 + tiles * sum(m > 32 for m in ms) <= 512
    W13, W2, Ws13, Ws2 = weights(c)
    out = torch.full((cfg.B, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    mb.moe_block(dev(c.X), dev(c.Wr), cfg.k, W13, W2, out, ws, Ws13, Ws2, dev(c.bias), c.bias_ld, ids, w)
    torch.cuda.synchronize()
    say("cut heaviest first: tasks uncut", t1, "variant", mb.last_variant())
    ref = c.oracle_block()["out"]
    g = host(out)
    assert np.array_equal(host(ids), c.ids)
    assert np.max(np.abs(host(w) - c.w)) <= 1e-5
    r_err, r_rnd = check_block_output(g, ref)
    say("  max|err|/rms %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
    assert r_rnd + 2e-3 <= 2e-2    # the stated bar applies here and was asserted
