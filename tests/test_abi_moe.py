"""CPU tests of the MoE chain's C entry points: the padded-row bound and workspace sizes, and the
host-side rejections of dispatch, gathered quantization, SwiGLU (with and without the
quantization), combine and the fused forward. Every case is rejected before any device call or
is a documented no-op (fake pointers are never dereferenced, nothing is launched)."""

import numpy as np
import pytest

from block_scaled_fp8_bfp8_amd import _native
from oracle import moe

E_INV = _native.BFP8_ERR_INVALID_ARGUMENT
E_UNS = _native.BFP8_ERR_UNSUPPORTED
E_MIS = _native.BFP8_ERR_MISALIGNED
E_WS = _native.BFP8_ERR_WORKSPACE

P1, P2, P3, P4, P5, P6, P7 = (0x10000000 * i for i in range(1, 8))  # fake, 256-byte aligned


@pytest.fixture(scope="module")
def lib():
    return _native.lib()


def test_padded_rows_bounds_every_layout(lib):
    """bfp8_moe_padded_rows(S, E, align) is a multiple of align and at least the padded size of
    any routing of S pairs over E experts (the oracle's layout), and equal to it when every
    expert holds one pair."""
    rng = np.random.default_rng(0)
    for s, e, align in [(1, 1, 128), (7, 3, 4), (64, 16, 128), (100, 8, 16), (5, 64, 128), (300, 7, 1)]:
        bound = lib.bfp8_moe_padded_rows(s, e, align)
        assert bound % align == 0
        for _ in range(20):
            ids = rng.integers(0, e, s).astype(np.int32).reshape(s, 1)
            _, _, layout, _ = moe.layout_ref(ids, e, align)
            assert layout.size <= bound
        if s <= e:  # one pair per expert: s blocks of align rows
            ids = np.arange(s, dtype=np.int32).reshape(s, 1)
            assert moe.layout_ref(ids, e, align)[2].size == s * align == bound
    for args in [(-1, 4, 128), (10, 0, 128), (10, 4, 0)]:
        assert lib.bfp8_moe_padded_rows(*args) == 0


def test_workspace_sizes(lib):
    assert lib.bfp8_moe_dispatch_workspace_bytes(0, 4) == 4 * 4  # the per-expert counters alone
    assert lib.bfp8_moe_dispatch_workspace_bytes(1024, 16) == (1 * 16 + 16) * 4
    assert lib.bfp8_moe_dispatch_workspace_bytes(1025, 16) == (2 * 16 + 16) * 4
    assert lib.bfp8_moe_dispatch_workspace_bytes(-1, 4) == 0
    small = lib.bfp8_moe_forward_workspace_bytes(512, 8, 16, 7168, 2048)
    rows = lib.bfp8_moe_padded_rows(512 * 8, 16, 128)
    # at least the tokens' codes, the up-projection output, the second codes and the down output
    assert small >= 512 * 7168 + rows * 2048 * 2 * 2 + rows * 2048 + rows * 7168 * 2
    assert small % 256 == 0
    for args in [(0, 8, 16, 7168, 2048), (512, 0, 16, 7168, 2048), (512, 8, 0, 7168, 2048), (1 << 29, 8, 16, 128, 128)]:
        assert lib.bfp8_moe_forward_workspace_bytes(*args) == 0


def _dispatch(lib, ids=P1, S=64, E=8, align=128, rop=P2, por=P3, lay=P4, start=P5, ws=P6, wsb=1 << 20):
    return lib.bfp8_moe_dispatch(ids, S, E, align, rop, por, lay, start, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(S=-1), E_INV), (dict(E=0), E_UNS), (dict(E=1025), E_UNS), (dict(align=0), E_INV),
    (dict(align=8192), E_INV), (dict(S=1 << 31, E=1024), E_UNS), (dict(ids=None), E_INV), (dict(rop=None), E_INV),
    (dict(por=None), E_INV), (dict(lay=None), E_INV), (dict(start=None), E_INV), (dict(S=0, start=None), E_INV),
    (dict(ids=P1 + 2), E_MIS), (dict(start=P5 + 1), E_MIS), (dict(ws=None), E_WS), (dict(wsb=8), E_WS),
    (dict(ws=P6 + 2), E_MIS),
])
def test_dispatch_rejections(lib, kw, status):
    assert _dispatch(lib, **kw) == status, lib.bfp8_last_error_message()


def _gather(lib, x=P1, dt=_native.BFP8_IN_BF16, src_rows=16, K=256, ldx=256, row_src=P2, div=2, M=32, q=P3,
            ldq=256, as_=P4, ld_as=32):
    return lib.bfp8_quant_act_gather(x, dt, src_rows, K, ldx, row_src, div, M, q, ldq, as_, ld_as, None)


@pytest.mark.parametrize("kw,status", [
    (dict(src_rows=0), E_INV), (dict(div=0), E_INV), (dict(row_src=None), E_INV), (dict(row_src=P2 + 2), E_MIS),
    (dict(M=-1), E_INV), (dict(dt=7), E_UNS), (dict(ld_as=31), E_INV), (dict(q=None), E_INV), (dict(ldq=128), E_INV),
])
def test_gather_rejections(lib, kw, status):
    assert _gather(lib, **kw) == status, lib.bfp8_last_error_message()


def test_gather_m_zero_is_a_no_op(lib):
    assert _gather(lib, M=0, row_src=None, src_rows=0) == _native.BFP8_OK


def _swiglu_quant(lib, proj=P1, M=64, I=256, ldp=512, lay=P2, q=P3, ldq=256, as_=P4, ld_as=64):
    return lib.bfp8_swiglu_quant(proj, M, I, ldp, lay, q, ldq, as_, ld_as, None)


def _swiglu(lib, proj=P1, M=64, I=256, ldp=512, lay=P2, h=P3, ldh=256):
    return lib.bfp8_swiglu(proj, M, I, ldp, lay, h, ldh, None)


_SWIGLU_COMMON = [
    (dict(M=-1), E_INV), (dict(I=0), E_UNS), (dict(I=200, ldp=400), E_UNS), (dict(I=1 << 31, ldp=1 << 32), E_UNS),
    (dict(M=1 << 31), E_UNS), (dict(proj=None), E_INV), (dict(ldp=511), E_INV), (dict(ldp=516), E_MIS),
    (dict(proj=P1 + 8), E_MIS), (dict(lay=P2 + 2), E_MIS),
]


@pytest.mark.parametrize("kw,status", _SWIGLU_COMMON + [
    (dict(q=None), E_INV), (dict(as_=None), E_INV), (dict(ldq=255), E_INV), (dict(ld_as=63), E_INV),
    (dict(ldq=264), E_MIS), (dict(q=P3 + 8), E_MIS), (dict(as_=P4 + 2), E_MIS),
])
def test_swiglu_quant_rejections(lib, kw, status):
    assert _swiglu_quant(lib, **kw) == status, lib.bfp8_last_error_message()


@pytest.mark.parametrize("kw,status", _SWIGLU_COMMON + [
    (dict(h=None), E_INV), (dict(ldh=255), E_INV), (dict(ldh=260), E_MIS), (dict(h=P3 + 8), E_MIS),
])
def test_swiglu_rejections(lib, kw, status):
    assert _swiglu(lib, **kw) == status, lib.bfp8_last_error_message()


def test_swiglu_m_zero_is_a_no_op(lib):
    assert _swiglu_quant(lib, M=0, proj=None, q=None, as_=None) == _native.BFP8_OK
    assert _swiglu(lib, M=0, proj=None, h=None) == _native.BFP8_OK


def _combine(lib, out=P1, ldo=256, rop=P2, w=P3, T=32, k=4, H=256, y=P4, ldy=256):
    return lib.bfp8_moe_combine(out, ldo, rop, w, T, k, H, y, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), E_INV), (dict(k=0), E_INV), (dict(H=0), E_UNS), (dict(H=12), E_UNS), (dict(T=1 << 30, k=4), E_UNS),
    (dict(out=None), E_INV), (dict(rop=None), E_INV), (dict(w=None), E_INV), (dict(y=None), E_INV),
    (dict(ldo=255), E_INV), (dict(ldy=128), E_INV), (dict(ldo=260), E_MIS), (dict(out=P1 + 8), E_MIS),
    (dict(rop=P2 + 2), E_MIS), (dict(w=P3 + 1), E_MIS),
])
def test_combine_rejections(lib, kw, status):
    assert _combine(lib, **kw) == status, lib.bfp8_last_error_message()


def test_combine_t_zero_is_a_no_op(lib):
    assert _combine(lib, T=0, out=None, rop=None, w=None, y=None) == _native.BFP8_OK


def _forward(lib, hidden=P1, T=32, H=256, ldh=256, ids=P2, w=P3, k=4, E=8, wu=P4, su=P5, wd=P6, sd=P7, I=128,
             y=0x7000000, ldy=256, ws=0x80000000, wsb=None):
    if wsb is None:
        wsb = lib.bfp8_moe_forward_workspace_bytes(T, k, E, H, I) if T > 0 else 0
    return lib.bfp8_moe_forward(hidden, T, H, ldh, ids, w, k, E, wu, su, wd, sd, I, y, ldy, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), E_INV), (dict(k=0), E_INV), (dict(E=0), E_UNS), (dict(E=2000), E_UNS), (dict(H=100), E_UNS),
    (dict(I=64), E_UNS), (dict(wu=None), E_INV), (dict(sd=None), E_INV), (dict(hidden=None), E_INV),
    (dict(ids=None), E_INV), (dict(w=None), E_INV), (dict(y=None), E_INV), (dict(ldh=128), E_MIS),
    (dict(hidden=P1 + 8), E_MIS), (dict(ws=None), E_WS), (dict(wsb=1024), E_WS), (dict(ws=0x80000000 + 128), E_MIS),
    (dict(ldy=128), E_INV), (dict(ids=P2 + 2), E_MIS),
])
def test_forward_rejections(lib, kw, status):
    assert _forward(lib, **kw) == status, lib.bfp8_last_error_message()


def test_forward_t_zero_is_a_no_op(lib):
    assert _forward(lib, T=0, hidden=None, ids=None, w=None, y=None, ws=None) == _native.BFP8_OK


def _gathered(lib, a=P1, lda=256, as_=P2, ld_as=128, rows=16, src=P3, div=2, b=P4, ldb=256, bs=P5, ld_bs=2, lay=P6,
              G=4, c=P7, ldc=64, M=128, N=64, K=256):
    return lib.bfp8_grouped_gemm_gathered(a, lda, as_, ld_as, rows, src, div, b, ldb, bs, ld_bs, lay, G, c, ldc, M, N,
                                          K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), E_INV), (dict(M=100), E_INV), (dict(M=1 << 31), E_UNS), (dict(rows=0), E_INV), (dict(div=0), E_INV),
    (dict(src=None), E_INV), (dict(src=P3 + 2), E_MIS), (dict(ld_as=15), E_INV), (dict(ld_as=100), E_INV),
    (dict(lda=128), E_INV),
    (dict(a=None), E_INV), (dict(as_=None), E_INV), (dict(c=None), E_INV), (dict(lay=None), E_INV),
    (dict(lay=P6 + 2), E_MIS), (dict(G=0), E_INV), (dict(ldc=32), E_INV), (dict(K=200), E_UNS), (dict(b=None), E_INV),
])
def test_grouped_gathered_rejections(lib, kw, status):
    assert _gathered(lib, **kw) == status, lib.bfp8_last_error_message()


def test_grouped_gathered_m_zero_is_a_no_op(lib):
    assert _gathered(lib, M=0, src=None, lay=None, rows=0) == _native.BFP8_OK


def _scatter(lib, x=P1, dt=_native.BFP8_IN_BF16, M=16, K=256, ldx=256, q=P2, ldq=256, as_=P3, ld_as=64, dst=P4, fan=4):
    return lib.bfp8_quant_act_scatter(x, dt, M, K, ldx, q, ldq, as_, ld_as, dst, fan, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), E_INV), (dict(dt=9), E_UNS), (dict(K=200), E_UNS), (dict(fan=0), E_INV), (dict(dst=None), E_INV),
    (dict(dst=P4 + 2), E_MIS), (dict(ld_as=8), E_INV), (dict(q=None), E_INV), (dict(as_=None), E_INV),
    (dict(M=1 << 29, fan=8, ld_as=1 << 30), E_UNS),
])
def test_quant_scatter_rejections(lib, kw, status):
    assert _scatter(lib, **kw) == status, lib.bfp8_last_error_message()


def test_quant_scatter_m_zero_is_a_no_op(lib):
    assert _scatter(lib, M=0, x=None, q=None, as_=None, dst=None) == _native.BFP8_OK
