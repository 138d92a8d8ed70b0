"""Seeded input generator: determinism, per-row streams, encoding, recipe."""
import hashlib

import numpy as np

from moe_block_skinny_amd import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_bf16_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, 3.0e38, 1e-40], np.float32)
    got = synth.to_bf16_bits(v)
    # 1+2^-8 is halfway between 1.0 and 1+2^-7: ties to even -> 1.0 (0x3F80);
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 0x3F82
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F62, 0x0001]


def test_determinism_and_independence():
    cfg = synth.CONFIGS["tp16_b8"]
    a = synth.x(cfg, 0)
    assert _h(a) == _h(synth.x(cfg, 0))
    assert _h(a) != _h(synth.x(cfg, 1))
    for t in range(cfg.B):
        assert np.array_equal(a[t], synth.x_row(cfg, 0, t))
    assert not np.array_equal(synth.x_row(cfg, 0, 3, 1), a[3])
    assert np.array_equal(synth.expert_w13(cfg, 0, 5), synth.expert_w13(cfg, 0, 5))
    assert not np.array_equal(synth.expert_w13(cfg, 0, 5), synth.expert_w13(cfg, 0, 6))


def test_shapes_and_scales():
    cfg = synth.CONFIGS["tp8_b64"]
    wide = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    w13 = synth.expert_w13(cfg, 0, 0)
    w2 = synth.expert_w2(cfg, 0, 0)
    assert w13.shape == (2 * cfg.I, cfg.d) and w13.dtype == np.uint16
    assert w2.shape == (cfg.d, cfg.I)
    assert abs(wide(w13).std() * np.sqrt(cfg.d) - 1) < 0.01
    assert abs(wide(w2).std() * np.sqrt(cfg.I) - 1) < 0.01
    assert synth.shared_w13(cfg, 0).shape == (2 * cfg.Is, cfg.d)
    tiny = synth.CONFIGS["tiny"]
    assert synth.router_w(tiny, 0).dtype == np.float32
    assert synth.shared_w13(tiny, 0) is None


def test_routing_biases():
    g = synth.CONFIGS["tp16_b8"]
    b, ld = synth.bias(g, 0)
    assert b.shape == (g.B, g.E) and ld == g.E
    many = np.concatenate([synth.gumbel_row(g, 0, t) for t in range(200)])
    assert abs(many.mean() - 0.5772156649) < 0.01      # Gumbel mean = Euler-Mascheroni
    z = synth.CONFIGS["tp8_b64"]
    b, ld = synth.bias(z, 0)
    assert b.shape == (z.E,) and ld == 0
    ranks = np.sort(np.round(np.exp(-b.astype(np.float64) / 1.1)).astype(int))
    assert np.array_equal(ranks, np.arange(1, z.E + 1))
    assert synth.bias(synth.CONFIGS["tp16_b1"], 0) == (None, 0)
