"""GPU parity over seeded random shapes: the automatic schedule and tile choices (K-split or tiled;
the tiled plans with their column splits and fewest-round shapes; the 1x64 kernel's three tile
shapes) on ragged M, N and K, each against the oracle on sampled rows, with output rows padded
so that columns past N can be checked untouched."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import quant
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20261203)


def _shapes(count):
    out = []
    for _ in range(count):
        m = int(_RNG.choice([_RNG.integers(1, 257), _RNG.integers(257, 4300)]))
        n = int(_RNG.integers(1, 4300))
        k = int(_RNG.integers(1, 262)) * 16
        out.append((m, n, k))
    return out


SHAPES = _shapes(12)
SHAPES_1X64 = _shapes(12)


def _rows(m, seed):
    if m <= 24:
        return np.arange(m)
    return np.unique(np.concatenate([[0, m - 1], np.random.default_rng(seed).choice(m, 22, replace=False)]))


def _padded_out(m, n, gpu):
    buf = torch.full((m, n + 5), -3.0, dtype=torch.bfloat16, device=gpu)
    return buf, buf[:, :n]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_random_shape(gpu, m, n, k):
    x = workloads.act_uniform(m, k, seed=m * 7 + k)
    q, s = bfp8.quant_act(x.to(gpu))
    q_ref, s_ref = quant.quant_act_ref(x.numpy())
    w = workloads.weight(n, k, seed=n * 3 + k)
    buf, out = _padded_out(m, n, gpu)
    announce("gemm random shape", m, n, k, "->", bfp8.schedule_for(m, n, k))
    bfp8.gemm(q, s, bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu), out=out)
    torch.cuda.synchronize()
    assert (buf[:, n:] == -3.0).all(), "columns past N were written"
    rows = _rows(m, m + n + k)
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    hw = tolerance.block_max_mass(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, np.arange(n)) if k < 128 else None
    tolerance.compare(bits(out)[rows], ref_bits, mass, k, f"gemm random {m}x{n}x{k}", hw_block=hw)


@pytest.mark.parametrize("m,n,k", SHAPES_1X64)
def test_gemm_1x64_random_shape(gpu, m, n, k):
    x = workloads.act_uniform(m, k, seed=m * 11 + k)
    q, s = bfp8.quant_act_1x64(x.to(gpu))
    q_ref, s_ref = quant.quant_act_ref(x.numpy(), group=64)
    w = workloads.weight_1x64(n, k, seed=n * 5 + k)
    buf, out = _padded_out(m, n, gpu)
    announce("gemm_1x64 random shape", m, n, k)
    bfp8.gemm_1x64(q, s, bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu), out=out)
    torch.cuda.synchronize()
    assert (buf[:, n:] == -3.0).all(), "columns past N were written"
    rows = _rows(m, m + n + k)
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows, k_block=64)
    hw = tolerance.block_max_mass(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, np.arange(n), 64) if k < 128 else None
    tolerance.compare(bits(out)[rows], ref_bits, mass, k, f"gemm_1x64 random {m}x{n}x{k}", hw_block=hw, k_block=64)
