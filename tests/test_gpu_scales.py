"""GPU parity of the scale-granularity adapter: per-tensor and per-token scales expanded to the
block grids bit for bit, and the block GEMM on them against the oracle's per-token product."""

import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
from block_scaled_fp8_bfp8_amd import _native
from oracle import scales
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return c


@pytest.mark.parametrize("m,k", [(1, 128), (37, 200), (300, 7168)])
def test_expanded_grids_bit_exact(gpu, m, k):
    rng = np.random.default_rng(m + k)
    s_tok = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    announce("expand_act_scales", m, k)
    got = bfp8.expand_act_scales(torch.from_numpy(s_tok).to(gpu), m, k)
    got_t = bfp8.expand_act_scales(torch.tensor([0.375], device=gpu), m, k)
    got_w = bfp8.expand_weight_scale(torch.tensor([3e-3], dtype=torch.float32, device=gpu), 300, k)
    torch.cuda.synchronize()
    assert got.stride(0) == 1 and got.shape == (m, -(-k // 128))
    np.testing.assert_array_equal(got.cpu().numpy(), scales.expand_act_scales_ref(s_tok, m, k))
    np.testing.assert_array_equal(got_t.cpu().numpy(), scales.expand_act_scales_ref(np.float32(0.375), m, k))
    np.testing.assert_array_equal(got_w.cpu().numpy(), scales.expand_weight_scale_ref(np.float32(3e-3), 300, k))


def test_padded_leading_dimension_untouched(gpu):
    m, k, ld = 5, 384, 9
    buf = torch.full((3, ld), -1.0, dtype=torch.float32, device=gpu)
    s = torch.arange(1, m + 1, dtype=torch.float32, device=gpu)
    announce("expand_act_scales padded", m, k, ld)
    st = _native.lib().bfp8_expand_act_scales(s.data_ptr(), 1, m, k, buf.data_ptr(), ld,
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == _native.BFP8_OK
    out = buf.cpu().numpy()
    assert (out[:, :m] == np.arange(1, m + 1)).all() and (out[:, m:] == -1.0).all()


@pytest.mark.parametrize("m,n,k", [(5, 576, 1024), (300, 640, 2048), (2048, 1024, 512)])
@pytest.mark.parametrize("per_token", [True, False])
def test_gemm_on_expanded_scales(gpu, m, n, k, per_token):
    """A per-token (or per-tensor) FP8 activation and a per-tensor FP8 weight through the block
    GEMM on expanded grids, against the oracle's per-token product."""
    rng = np.random.default_rng(m * 3 + n + k + per_token)
    a, b = _codes(rng, (m, k)), _codes(rng, (n, k))
    s_a = rng.uniform(1e-3, 2.0, m).astype(np.float32) if per_token else np.float32(0.5)
    s_b = np.float32(2e-3)
    announce("gemm on expanded scales", m, n, k, "per-token" if per_token else "per-tensor")
    sa_dev = torch.from_numpy(np.atleast_1d(s_a)).to(gpu)
    a_s = bfp8.expand_act_scales(sa_dev, m, k)
    b_s = bfp8.expand_weight_scale(torch.tensor([float(s_b)], dtype=torch.float32, device=gpu), n, k)
    c = bfp8.gemm(torch.from_numpy(a).to(gpu), a_s, torch.from_numpy(b).to(gpu), b_s)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 24 else np.unique(np.concatenate([[0, m - 1], rng.choice(m, 22, replace=False)]))
    want = scales.gemm_per_token_ref(a[rows], s_a[rows] if per_token else s_a, b, s_b)
    a_s_ref = scales.expand_act_scales_ref(s_a, m, k)
    b_s_ref = scales.expand_weight_scale_ref(s_b, n, k)
    cols = np.arange(n)
    mag = tolerance.masses(a, a_s_ref, b, b_s_ref, rows, cols)
    # codes drawn over the whole e4m3 range: the hardware block-dot term of the tolerance applies
    mmax = tolerance.block_max_mass(a, a_s_ref, b, b_s_ref, rows, cols)
    st = tolerance.compare(bits(c)[rows], want, mag, k, f"expanded scales {m}x{n}x{k}", hw_block=mmax)
    print(st)
