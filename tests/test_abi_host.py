"""C-ABI library on the host, no GPU: it loads, exports every symbol the
public header declares, sizes workspaces and plans, and rejects every bad
argument with the documented status before touching HIP.

Fake device pointers are only ever passed to calls that must fail
validation, so no kernel is launched here.
"""
import os
import re

import pytest

from moe_block_skinny_amd import binding as mb
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000          # an aligned fake device address (never dereferenced)
MIS = A + 4          # misaligned
BIG = 1 << 34        # "large enough" workspace byte count
lib = mb.lib


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe_skinny.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_exports_every_declared_symbol():
    names = header_functions()
    assert "moe_route" in names and "skinny_gemm" in names and len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(mb.SIGNATURES) == set(names)
    assert lib.moe_abi_version() == 1


@pytest.mark.parametrize("B,k,E", [(1, 2, 16), (1, 8, 384), (8, 8, 384), (64, 8, 384), (3, 4, 5)])
def test_plan_words_match_oracle(B, k, E):
    assert lib.moe_plan_words(B, k, E) == orc.plan_words(B, k, E)


def test_workspace_bytes():
    f = mb.workspace_bytes
    r1 = f(mb.OP_ROUTE, mb.DT_BF16, B=1, d=7168, E=384, k=8)
    r64 = f(mb.OP_ROUTE, mb.DT_BF16, B=64, d=7168, E=384, k=8)
    assert 0 < r1 <= r64 and r1 % 256 == 0
    assert f(mb.OP_EXPERT_FFN, mb.DT_BF16, B=64, d=7168, E=384, k=8, I=256, Is=256) >= (512 + 64) * 256 * 4
    blk = f(mb.OP_BLOCK, mb.DT_BF16, B=8, d=7168, E=384, k=8, I=128, Is=128)
    assert blk >= f(mb.OP_ROUTE, mb.DT_BF16, B=8, d=7168, E=384, k=8) + (8 * 8 + 8) * 128 * 4
    # the dense product: no workspace for fp32 (vector shapes only); bf16
    # sizes the MFMA shape's K-slice partial sums (fp32 [slices][B][N])
    assert f(mb.OP_SKINNY_GEMM, mb.DT_F32, B=8, N=3072, K=7168) == 0
    assert f(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=64, N=3072, K=7168) >= 2 * 64 * 3072 * 4


def test_status_str():
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(3) == b"workspace too small"


def gemm(**kw):
    a = dict(dt=mb.DT_BF16, B=4, N=64, K=256, X=A, W=A, Y=A, ydt=mb.DT_BF16, ws=A, wsb=BIG)
    a.update(kw)
    return lib.skinny_gemm(a["dt"], a["B"], a["N"], a["K"], a["X"], a["W"], a["Y"], a["ydt"],
                           a["ws"], a["wsb"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), mb.EINVAL),
    (dict(ydt=7), mb.EINVAL),
    (dict(B=0), mb.EINVAL),
    (dict(N=-1), mb.EINVAL),
    (dict(X=None), mb.EINVAL),
    (dict(W=MIS), mb.EINVAL),
    (dict(Y=MIS), mb.EINVAL),
    (dict(B=65), mb.EUNSUPPORTED),
    (dict(K=252), mb.EUNSUPPORTED),
    (dict(dt=mb.DT_F32, ydt=mb.DT_F32, B=16), mb.EUNSUPPORTED),
    (dict(B=16, K=264), mb.EUNSUPPORTED),
])
def test_skinny_gemm_validation(kw, status):
    assert gemm(**kw) == status
    assert lib.moe_last_error() != b""


def gemm_residual(**kw):
    a = dict(dt=mb.DT_BF16, B=4, N=64, K=256, X=A, W=A, R=A, Y=A, ydt=mb.DT_BF16, ws=A, wsb=BIG)
    a.update(kw)
    return lib.skinny_gemm_residual(a["dt"], a["B"], a["N"], a["K"], a["X"], a["W"], a["R"], a["Y"],
                                    a["ydt"], a["ws"], a["wsb"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(R=None), mb.EINVAL),
    (dict(R=MIS), mb.EINVAL),
    (dict(dt=7), mb.EINVAL),
    (dict(X=None), mb.EINVAL),
    (dict(B=65), mb.EUNSUPPORTED),
    (dict(K=252), mb.EUNSUPPORTED),
])
def test_skinny_gemm_residual_validation(kw, status):
    assert gemm_residual(**kw) == status
    assert lib.moe_last_error() != b""


def route(**kw):
    a = dict(dt=mb.DT_BF16, B=8, d=7168, E=384, k=8, X=A, Wr=A, bias=None, ld=0, ids=A, w=A,
             plan=A, lo=None, ws=A, wsb=BIG)
    a.update(kw)
    return lib.moe_route(a["dt"], a["B"], a["d"], a["E"], a["k"], a["X"], a["Wr"], a["bias"],
                         a["ld"], a["ids"], a["w"], a["plan"], a["lo"], a["ws"], a["wsb"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), mb.EINVAL),
    (dict(k=9, E=8), mb.EINVAL),
    (dict(B=0), mb.EINVAL),
    (dict(B=65), mb.EUNSUPPORTED),
    (dict(E=513, k=8), mb.EUNSUPPORTED),
    (dict(k=17), mb.EUNSUPPORTED),
    (dict(d=7160), mb.EUNSUPPORTED),
    (dict(dt=mb.DT_F32, B=9, d=1024), mb.EUNSUPPORTED),
    (dict(X=MIS), mb.EINVAL),
    (dict(plan=None), mb.EINVAL),
    (dict(bias=A, ld=7), mb.EINVAL),
    (dict(bias=MIS), mb.EINVAL),
    (dict(lo=MIS), mb.EINVAL),
    (dict(wsb=1024), mb.EWORKSPACE),
])
def test_route_validation(kw, status):
    assert route(**kw) == status


def ffn(**kw):
    a = dict(dt=mb.DT_BF16, B=8, d=7168, E=384, k=8, I=128, X=A, plan=A, W13=A, W2=A, Is=128,
             Ws13=A, Ws2=A, Y=A, ws=A, wsb=BIG)
    a.update(kw)
    return lib.moe_expert_ffn(a["dt"], a["B"], a["d"], a["E"], a["k"], a["I"], a["X"], a["plan"],
                              a["W13"], a["W2"], a["Is"], a["Ws13"], a["Ws2"], a["Y"], a["ws"],
                              a["wsb"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(I=0), mb.EINVAL),
    (dict(I=100), mb.EUNSUPPORTED),
    (dict(I=288), mb.EUNSUPPORTED),
    (dict(Is=96 + 8), mb.EUNSUPPORTED),
    (dict(Ws2=None), mb.EINVAL),
    (dict(W2=MIS), mb.EINVAL),
    (dict(Y=None), mb.EINVAL),
    (dict(dt=mb.DT_F32, d=1024, I=512), mb.EUNSUPPORTED),
    (dict(wsb=4096), mb.EWORKSPACE),
])
def test_expert_ffn_validation(kw, status):
    assert ffn(**kw) == status


def test_combine_and_block_validation():
    assert lib.moe_combine(mb.DT_BF16, 0, 7168, 8, A, A, 1, A, 0) == mb.EINVAL
    assert lib.moe_combine(mb.DT_BF16, 65, 7168, 8, A, A, 1, A, 0) == mb.EUNSUPPORTED
    assert lib.moe_combine(mb.DT_BF16, 1, 7168, 8, A, MIS, 1, A, 0) == mb.EINVAL
    blk = lambda **kw: lib.moe_block(
        kw.get("dt", mb.DT_BF16), kw.get("B", 1), 7168, 384, 8, 128, 128, A, A, None, 0, A, A,
        A, A, kw.get("out", A), None, None, A, kw.get("wsb", BIG), 0)
    assert blk(B=65) == mb.EUNSUPPORTED
    assert blk(out=MIS) == mb.EINVAL
    assert blk(wsb=1000) == mb.EWORKSPACE


def test_forced_variant_scope():
    prev = mb.set_variant("gemv")
    try:
        assert gemm(B=4) == mb.EUNSUPPORTED
        assert b"gemv" in lib.moe_last_error()
        assert route(B=3) == mb.EUNSUPPORTED
        mb.set_variant("splitk")
        assert gemm(B=9) == mb.EUNSUPPORTED
        assert ffn(B=9) == mb.EUNSUPPORTED
        mb.set_variant("mfma")
        assert gemm(dt=mb.DT_F32, ydt=mb.DT_F32, B=2) == mb.EUNSUPPORTED
        assert gemm(B=2, K=264) == mb.EUNSUPPORTED
        mb.set_variant("rows")
        assert gemm(B=9) == mb.EUNSUPPORTED
        assert gemm(dt=mb.DT_F32, ydt=mb.DT_F32, B=2) == mb.EUNSUPPORTED
        assert gemm(B=2, K=8200) == mb.EUNSUPPORTED
        assert b"rows" in lib.moe_last_error()
    finally:
        mb.set_variant(prev)
    assert mb.set_variant(prev) == prev


def route_latent(**kw):
    a = dict(dt=mb.DT_BF16, B=8, d=7168, E=384, k=8, L=1024, X=A, Wr=A, Wl=A, bias=None, ld=0, ids=A, w=A,
             plan=A, lat=A, ldt=mb.DT_BF16, lo=None, ws=A, wsb=BIG)
    a.update(kw)
    return lib.moe_route_latent(a["dt"], a["B"], a["d"], a["E"], a["k"], a["L"], a["X"], a["Wr"], a["Wl"],
                                a["bias"], a["ld"], a["ids"], a["w"], a["plan"], a["lat"], a["ldt"], a["lo"],
                                a["ws"], a["wsb"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), mb.EINVAL),
    (dict(L=24), mb.EUNSUPPORTED),
    (dict(L=8208), mb.EUNSUPPORTED),
    (dict(E=382), mb.EUNSUPPORTED),
    (dict(ldt=7), mb.EINVAL),
    (dict(Wl=None), mb.EINVAL),
    (dict(lat=MIS), mb.EINVAL),
    (dict(B=65), mb.EUNSUPPORTED),
    (dict(wsb=4096), mb.EWORKSPACE),
])
def test_route_latent_validation(kw, status):
    assert route_latent(**kw) == status


def test_route_latent_workspace_covers_the_latent_rows():
    f = mb.workspace_bytes
    assert f(mb.OP_ROUTE_LATENT, mb.DT_BF16, B=64, d=7168, E=384, k=8, N=1024) > \
        f(mb.OP_ROUTE, mb.DT_BF16, B=64, d=7168, E=384, k=8)
