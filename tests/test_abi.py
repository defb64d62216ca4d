"""CPU tests of the C ABI: the library loads, exports every declared symbol, and rejects
invalid arguments on the host before any HIP call (fake pointers are never dereferenced)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

from block_scaled_fp8_bfp8_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp8.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bfp8_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _native.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared_functions()
    assert len(names) >= 10
    bound = {n for n, _, _ in _native.SIGNATURES}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
        assert n in bound, f"{n} has no ctypes signature"
    assert bound == set(names)


def test_version_and_status_strings(lib):
    assert lib.bfp8_abi_version() == 15
    for code, name in [(0, b"BFP8_OK"), (1, b"BFP8_ERR_INVALID_ARGUMENT"), (2, b"BFP8_ERR_UNSUPPORTED"),
                       (3, b"BFP8_ERR_MISALIGNED"), (4, b"BFP8_ERR_WORKSPACE"), (5, b"BFP8_ERR_DEVICE"),
                       (6, b"BFP8_ERR_LAUNCH")]:
        assert lib.bfp8_status_string(code) == name
    assert lib.bfp8_status_string(99) == b"BFP8_UNKNOWN_STATUS"
    assert lib.bfp8_gemm_workspace_bytes(4096, 4096, 4096) == 0


A = 0x10000000  # fake, 256-byte aligned device addresses: validation never dereferences them
AS = 0x20000000
B = 0x30000000
BS = 0x40000000
C = 0x50000000


def _gemm(lib, a=A, lda=256, as_=AS, ld_as=8, b=B, ldb=256, bs=BS, ld_bs=2, c=C, ldc=64, M=8, N=64, K=256,
          ws=None, wsb=0):
    return lib.bfp8_gemm(a, lda, as_, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(N=0), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=0), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=200, lda=256, ldb=256), _native.BFP8_ERR_UNSUPPORTED),
    (dict(K=144, lda=144, ldb=256), _native.BFP8_ERR_INVALID_ARGUMENT),  # rows must hold ceil(K/128) blocks
    (dict(K=144, lda=256, ldb=160), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=144, lda=256, ldb=256, ld_bs=1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(M=1 << 31), _native.BFP8_ERR_UNSUPPORTED),
    (dict(a=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(b=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(bs=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(c=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(lda=128), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldb=255), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_as=7), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_bs=1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldc=63), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(lda=264), _native.BFP8_ERR_MISALIGNED),
    (dict(ldb=260), _native.BFP8_ERR_MISALIGNED),
    (dict(a=A + 8), _native.BFP8_ERR_MISALIGNED),
    (dict(b=B + 1), _native.BFP8_ERR_MISALIGNED),
    (dict(as_=AS + 2), _native.BFP8_ERR_MISALIGNED),
    (dict(bs=BS + 1), _native.BFP8_ERR_MISALIGNED),
    (dict(c=C + 1), _native.BFP8_ERR_MISALIGNED),
    (dict(N=(1 << 24) + 1, ldb=256, ldc=(1 << 24) + 1), _native.BFP8_ERR_UNSUPPORTED),  # B spans 4 GiB + 256 B
    (dict(M=(1 << 24) + 1, lda=256, ld_as=(1 << 24) + 1), _native.BFP8_ERR_UNSUPPORTED),  # A likewise
    # 2^18 x 2^17 output tiles of 64 x 128: more than a 32-bit grid, though A and B span 2 GiB each
    (dict(M=1 << 24, N=1 << 24, K=128, lda=128, ldb=128, ld_as=1 << 24, ld_bs=1, ldc=1 << 24),
     _native.BFP8_ERR_UNSUPPORTED),
])
def test_gemm_rejections(lib, kw, status):
    st = _gemm(lib, **kw)
    assert st == status, lib.bfp8_last_error_message()
    assert len(lib.bfp8_last_error_message()) > 0


def test_m_zero_is_ok_without_device(lib):
    # M = 0 returns before any HIP call; a, as and c may be NULL
    assert _gemm(lib, M=0, a=None, as_=None, c=None, ld_as=0) == _native.BFP8_OK
    assert lib.bfp8_last_error_message() == b""


def _quant(lib, x=A, dt=0, M=4, K=256, ldx=256, q=B, ldq=256, as_=AS, ld_as=4):
    return lib.bfp8_quant_act(x, dt, M, K, ldx, q, ldq, as_, ld_as, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), _native.BFP8_ERR_UNSUPPORTED),
    (dict(M=-3), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=130, ldx=256, ldq=256), _native.BFP8_ERR_UNSUPPORTED),
    (dict(x=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldx=255), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldq=128), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_as=3), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldx=258, dt=1), _native.BFP8_ERR_MISALIGNED),
    (dict(ldq=264), _native.BFP8_ERR_MISALIGNED),
    (dict(x=A + 4), _native.BFP8_ERR_MISALIGNED),
    (dict(q=B + 8), _native.BFP8_ERR_MISALIGNED),
    (dict(as_=AS + 1), _native.BFP8_ERR_MISALIGNED),
])
def test_quant_rejections(lib, kw, status):
    assert _quant(lib, **kw) == status, lib.bfp8_last_error_message()


def test_quant_m_zero_ok(lib):
    assert _quant(lib, M=0, x=None, q=None, as_=None) == _native.BFP8_OK


def _grouped(lib, a=A, lda=256, as_=AS, ld_as=128, b=B, ldb=256, bs=BS, ld_bs=2, lay=0x60000000, G=2, c=C,
             ldc=64, M=128, N=64, K=256):
    return lib.bfp8_grouped_gemm_contiguous(a, lda, as_, ld_as, b, ldb, bs, ld_bs, lay, G, c, ldc, M, N, K, None, 0,
                                            None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=100, ld_as=128), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(G=0), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(lay=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(lay=0x60000002), _native.BFP8_ERR_MISALIGNED),
    (dict(K=200), _native.BFP8_ERR_UNSUPPORTED),
    (dict(K=192, lda=192), _native.BFP8_ERR_INVALID_ARGUMENT),  # A rows must hold two whole blocks
    (dict(ldc=32), _native.BFP8_ERR_INVALID_ARGUMENT),
])
def test_grouped_rejections(lib, kw, status):
    assert _grouped(lib, **kw) == status, lib.bfp8_last_error_message()


def test_schedule_override(lib):
    try:
        assert lib.bfp8_set_schedule(7) == _native.BFP8_ERR_INVALID_ARGUMENT
        assert lib.bfp8_get_schedule() == 0
        assert lib.bfp8_gemm_schedule_for(1, 4096, 4096) == 1
        assert lib.bfp8_gemm_schedule_for(4096, 4096, 4096) == 2
        assert lib.bfp8_set_schedule(2) == 0
        assert lib.bfp8_gemm_schedule_for(1, 4096, 4096) == 2
        assert lib.bfp8_set_schedule(4) == _native.BFP8_ERR_INVALID_ARGUMENT
        assert lib.bfp8_set_schedule(3) == 0  # persistent: only by override
        assert lib.bfp8_gemm_schedule_for(8192, 4096, 4096) == 3
        assert lib.bfp8_gemm_workspace_bytes(8192, 4096, 4096) == 0
        assert lib.bfp8_linear_fuses(1, 4096, 4096, 4096) == 0
    finally:
        lib.bfp8_set_schedule(0)
    for m in (8192, 7680, 16384, 2048):  # the automatic choice never runs the persistent kernel
        assert lib.bfp8_gemm_schedule_for(m, 4096, 4096) == 2


def test_schedule_by_shape(lib):
    """Automatic choice, from the two schedules' time models: K-split at small M on the square
    weight and on the hidden-5120 o_proj / down weights up to M = 128; the tiled schedule above
    256 rows, on o_proj / down at M = 256, and at M >= 64 on the 51200-wide gate+up weight, where
    the K-split copies re-read each weight strip per 32-64 rows (measured 1.1-2.2x slower)."""
    small, tiled = 1, 2
    for m in (1, 16, 64, 128, 256):
        assert lib.bfp8_gemm_schedule_for(m, 4096, 4096) == small
    for m in (1, 16, 64, 128):
        assert lib.bfp8_gemm_schedule_for(m, 5120, 25600) == small
        assert lib.bfp8_gemm_schedule_for(m, 5120, 8192) == small
    for m in (1, 16):
        assert lib.bfp8_gemm_schedule_for(m, 51200, 5120) == small
    for m in (64, 128, 256):
        assert lib.bfp8_gemm_schedule_for(m, 51200, 5120) == tiled
    assert lib.bfp8_gemm_schedule_for(256, 5120, 25600) == tiled
    assert lib.bfp8_gemm_schedule_for(256, 5120, 8192) == tiled
    for n, k in ((4096, 4096), (576, 7168), (51200, 5120)):
        assert lib.bfp8_gemm_schedule_for(257, n, k) == tiled


def _linear(lib, x=A, dt=1, M=8, K=256, ldx=256, b=B, ldb=256, bs=BS, ld_bs=2, bias=None, c=C, ldc=64, N=64,
            ws=0x70000000, wsb=None):
    if wsb is None:
        wsb = lib.bfp8_linear_workspace_bytes(M, N, K) if M >= 0 else 0
    return lib.bfp8_linear(x, dt, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, ws, wsb, None)


def test_linear_workspace_size(lib):
    # quantized codes (M x K bytes), then float32 scales (M x K/128), each region a whole number of
    # 256-byte units; the GEMM itself needs none
    assert lib.bfp8_linear_workspace_bytes(8, 64, 256) == 2048 + 256
    assert lib.bfp8_linear_workspace_bytes(3, 64, 384) == 1280 + 256
    assert lib.bfp8_linear_workspace_bytes(0, 64, 256) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(dt=0), _native.BFP8_ERR_UNSUPPORTED),
    (dict(bias=0x80000001), _native.BFP8_ERR_MISALIGNED),
    (dict(ws=0x70000010), _native.BFP8_ERR_MISALIGNED),
    (dict(wsb=1024), _native.BFP8_ERR_WORKSPACE),
    (dict(ws=None), _native.BFP8_ERR_WORKSPACE),
    (dict(M=-1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=200, ldx=256), _native.BFP8_ERR_UNSUPPORTED),
    (dict(x=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(x=A + 2), _native.BFP8_ERR_MISALIGNED),
    (dict(ldx=100), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ldc=32), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_bs=1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(b=None), _native.BFP8_ERR_INVALID_ARGUMENT),
])
def test_linear_rejections(lib, kw, status):
    assert _linear(lib, **kw) == status, lib.bfp8_last_error_message()
    assert len(lib.bfp8_last_error_message()) > 0


def test_linear_m_zero_ok_without_device(lib):
    assert _linear(lib, M=0, x=None, ws=None, wsb=0) == _native.BFP8_OK


def _linear_noalloc(lib, x=A, dt=1, M=8, K=256, ldx=256, b=B, ldb=256, bs=BS, ld_bs=2, bias=None, c=C, ldc=64, N=64):
    return lib.bfp8_linear_noalloc(x, dt, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=2048, K=40960, ldx=40960, ldb=40960, ld_bs=320), _native.BFP8_ERR_UNSUPPORTED),  # staging > 64 MiB
    (dict(M=-1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=200, ldx=256, ldb=256), _native.BFP8_ERR_UNSUPPORTED),
    (dict(dt=0, M=0), _native.BFP8_ERR_UNSUPPORTED),
])
def test_linear_noalloc_rejections_on_the_host(lib, kw, status):
    assert _linear_noalloc(lib, **kw) == status, lib.bfp8_last_error_message()
    assert len(lib.bfp8_last_error_message()) > 0


def test_linear_noalloc_limit(lib):
    # the largest layer at M = 2048 whose staging fits 64 MiB, and one K block more
    assert lib.bfp8_linear_workspace_bytes(2048, 64, 30720) <= 64 << 20
    assert lib.bfp8_linear_workspace_bytes(2048, 64, 32768) > 64 << 20
    assert _linear_noalloc(lib, M=2048, K=32768, ldx=32768, ldb=32768, ld_bs=256) == _native.BFP8_ERR_UNSUPPORTED
    assert _linear_noalloc(lib, M=0, x=None) == _native.BFP8_OK


def _gemm_e8(lib, a=A, lda=256, as_=AS, ld_as=8, b=B, ldb=256, bs=BS, ld_bs=4, c=C, ldc=64, M=8, N=64, K=256):
    return lib.bfp8_gemm_ue8m0(a, lda, as_, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ld_as=9), _native.BFP8_ERR_MISALIGNED),
    (dict(ld_bs=2), _native.BFP8_ERR_MISALIGNED),
    (dict(ld_bs=6), _native.BFP8_ERR_MISALIGNED),
    (dict(as_=AS + 2), _native.BFP8_ERR_MISALIGNED),
    (dict(bs=BS + 1), _native.BFP8_ERR_MISALIGNED),
    (dict(ld_as=4), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=200), _native.BFP8_ERR_UNSUPPORTED),
    (dict(bs=None), _native.BFP8_ERR_INVALID_ARGUMENT),
])
def test_gemm_ue8m0_rejections(lib, kw, status):
    assert _gemm_e8(lib, **kw) == status, lib.bfp8_last_error_message()


def test_ue8m0_m_zero_and_grouped(lib):
    assert _gemm_e8(lib, M=0, a=None, as_=None, c=None) == _native.BFP8_OK
    st = lib.bfp8_grouped_gemm_contiguous_ue8m0(A, 256, AS, 130, B, 256, BS, 4, 0x60000000, 2, C, 64, 128, 64, 256,
                                                None, 0, None)
    assert st == _native.BFP8_ERR_MISALIGNED, lib.bfp8_last_error_message()


def test_quant_ue8m0_accepts_byte_aligned_scales(lib):
    # one-byte codes need no alignment and any ld_as >= M; M = 0 is a no-op
    assert lib.bfp8_quant_act_ue8m0(A, 0, 0, 256, 256, B, 256, None, 0, None) == _native.BFP8_OK
    assert lib.bfp8_quant_act_ue8m0(A, 0, 4, 256, 256, B, 256, AS, 3, None) == _native.BFP8_ERR_INVALID_ARGUMENT


def _gpu_count():
    import torch

    return torch.cuda.device_count()


@pytest.mark.skipif(_gpu_count() > 0, reason="a GPU is visible: a valid call with fake pointers would launch")
@pytest.mark.parametrize("call", ["gemm", "linear"])
def test_valid_call_without_gpu_reports_device_error(lib, call):
    st = _gemm(lib) if call == "gemm" else _linear(lib)
    assert st in (_native.BFP8_ERR_DEVICE, _native.BFP8_ERR_UNSUPPORTED), lib.bfp8_last_error_message()
    assert b"hip" in lib.bfp8_last_error_message().lower() or b"device" in lib.bfp8_last_error_message().lower()


def test_missing_library_fails_loudly(tmp_path):
    code = ("import block_scaled_fp8_bfp8_amd._native as n; n.LIB_PATH = '/nonexistent/libbfp8.so'\n"
            "try:\n    n.lib()\nexcept n.LibraryMissing as e:\n    print('missing:', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert "missing:" in out.stdout and "no fallback" in out.stdout


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "block_scaled_fp8_bfp8_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(K=0), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(s_stride=-1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_as=3), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(s=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(as_=AS + 2), _native.BFP8_ERR_MISALIGNED),
])
def test_expand_act_scales_rejections(lib, kw, status):
    a = dict(s=BS, s_stride=1, M=4, K=256, as_=AS, ld_as=4)
    a.update(kw)
    assert lib.bfp8_expand_act_scales(a["s"], a["s_stride"], a["M"], a["K"], a["as_"], a["ld_as"], None) == status
    assert lib.bfp8_expand_act_scales(BS, 1, 0, 256, None, 0, None) == _native.BFP8_OK  # M = 0: no-op


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(ld_bs=1), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(bs=None), _native.BFP8_ERR_INVALID_ARGUMENT),
    (dict(s=BS + 1), _native.BFP8_ERR_MISALIGNED),
])
def test_expand_weight_scale_rejections(lib, kw, status):
    a = dict(s=BS, N=300, K=256, bs=AS, ld_bs=2)
    a.update(kw)
    assert lib.bfp8_expand_weight_scale(a["s"], a["N"], a["K"], a["bs"], a["ld_bs"], None) == status


PROBES_HEADER = os.path.join(ROOT, "include", "bfp8_probes.h")


def test_probe_library_exports_its_header():
    """The benchmark's probe library (its own .so, outside the GEMM path) exports and binds every
    function its header declares, and rejects bad arguments before launching anything."""
    text = re.sub(r"/\*.*?\*/", "", open(PROBES_HEADER).read(), flags=re.S)
    names = set(re.findall(r"\b(bfp8_probe_\w+)\s*\(", text))
    pr = _native.probes()
    assert names == {n for n, _, _ in _native.PROBE_SIGNATURES}
    for n in names:
        assert hasattr(pr, n), f"{n} not exported"
    assert pr.bfp8_probe_mfma_loop_flops(256, 2000) == 256 * 8 * 2000 * 8 * 2.0 * 16 * 16 * 128
    fake = 1 << 40
    assert pr.bfp8_probe_mfma_loop(fake, 256, 10, 3, None) == 1  # unknown mode
    assert pr.bfp8_probe_mfma_loop(None, 256, 10, 0, None) == 1
    assert pr.bfp8_probe_mfma32_loop_flops(256, 2000) == 256 * 8 * 2000 * 4 * 2.0 * 32 * 32 * 64
    assert pr.bfp8_probe_mfma32_loop(fake, 256, 10, 2, None) == 1  # unknown mode
    assert pr.bfp8_probe_mfma32_loop(None, 256, 10, 0, None) == 1
    assert pr.bfp8_probe_stream_read(fake + 8, 1 << 20, fake, 64, None) == 1  # misaligned source
    assert pr.bfp8_probe_stream_read(fake, 1000, fake, 64, None) == 1  # not whole 16-byte words
    assert pr.bfp8_probe_copy_lds(fake, 3, 64, 8, 1, fake, 1, None) == 1  # groups not a power of two
    assert pr.bfp8_probe_copy_lds(fake, 4, 60, 8, 1, fake, 1, None) == 1  # iters not a multiple of inflight
    assert pr.bfp8_probe_copy_lds(fake, 4, 64, 16, 2, fake, 1, None) == 1  # wide rows need inflight 8
    assert pr.bfp8_probe_copy_lds(fake, 4, 64, 8, 5, fake, 1, None) == 1
    assert pr.bfp8_probe_copy_lds(fake, 4, 64, 8, -1, fake, 1, None) == 1


def test_linear_fusion_choice(lib):
    """The linear layer quantizes inside the GEMM at small M, N and K on the K-split 16 x 16 tile,
    and only while the activation rows fit 32-bit copy offsets; a forced tiled schedule never
    fuses."""
    assert lib.bfp8_linear_fuses(1, 4096, 4096, 4096) == 1
    assert lib.bfp8_linear_fuses(1, 51200, 5120, 5120) == 1  # M = 1: every shape
    assert lib.bfp8_linear_fuses(1, 5120, 25600, 25600) == 1
    assert lib.bfp8_linear_fuses(4, 4096, 8192, 8192) == 1  # N * K = 2^25
    assert lib.bfp8_linear_fuses(4, 5120, 8192, 8192) == 0
    assert lib.bfp8_linear_fuses(8, 4096, 4096, 4096) == 1  # N * K = 2^24
    assert lib.bfp8_linear_fuses(8, 5120, 4096, 4096) == 0
    assert lib.bfp8_linear_fuses(9, 64, 1024, 1024) == 0
    assert lib.bfp8_linear_fuses(16, 4096, 4096, 4096) == 0
    assert lib.bfp8_linear_fuses(4, 4096, 4096, (1 << 30) + 64) == 0  # 3 rows of 2 GiB past row 0
    assert lib.bfp8_linear_fuses(1, 4096, 4096, (1 << 30) + 64) == 1  # one row: no row offset
    assert lib.bfp8_linear_fuses(0, 4096, 4096, 4096) == 0
    assert lib.bfp8_linear_fuses(4, 4096, 4100, 4100) == 0  # K not a multiple of 16
    assert lib.bfp8_linear_fuses(4, 4096, 4096, 4000) == 0  # ldx < K
    try:
        assert lib.bfp8_set_schedule(2) == _native.BFP8_OK  # tiled
        assert lib.bfp8_linear_fuses(1, 4096, 4096, 4096) == 0
        assert lib.bfp8_set_schedule(1) == _native.BFP8_OK  # small_m
        assert lib.bfp8_linear_fuses(1, 4096, 4096, 4096) == 1
    finally:
        lib.bfp8_set_schedule(0)


def test_gemm_1x64_rejections(lib):
    """The 1x64 GEMM validates as bfp8_gemm, plus ld_bs >= ceil(K/64) (weight scales of 64-wide
    K blocks); M = 0 is a no-op."""
    args = dict(a=A, lda=256, as_=AS, ld_as=8, b=B, ldb=256, bs=BS, ld_bs=4, c=C, ldc=64, M=8, N=64, K=208)
    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.bfp8_gemm_1x64(a["a"], a["lda"], a["as_"], a["ld_as"], a["b"], a["ldb"], a["bs"], a["ld_bs"],
                                  a["c"], a["ldc"], a["M"], a["N"], a["K"], None)
    assert call(ld_bs=3) == _native.BFP8_ERR_INVALID_ARGUMENT  # ceil(208/64) = 4
    assert call(ld_as=7) == _native.BFP8_ERR_INVALID_ARGUMENT
    assert call(K=100) == _native.BFP8_ERR_UNSUPPORTED  # K % 16
    assert call(lda=128) == _native.BFP8_ERR_INVALID_ARGUMENT  # rows of whole 128-byte blocks
    assert call(M=0) == _native.BFP8_OK
    assert lib.bfp8_quant_act_1x64(A, 1, 4, 208, 208, B, 256, AS, 3, None) == _native.BFP8_ERR_INVALID_ARGUMENT
    assert lib.bfp8_quant_act_1x64(A, 1, 0, 208, 208, B, 256, AS, 3, None) == _native.BFP8_OK
