"""GPU parity of the 1x64 / 128x64 layout: the quantizer with 64-wide groups (bit-exact against
the oracle) and the GEMM with 64-wide K scale blocks (against the oracle under the float32
floor with K/64 promotions), on every K-split tile, ragged N, K tails where the last 128-wide
block holds one full, one partial or no second group, large M on sampled rows, and run-to-run
determinism."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import quant
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu


def _quant_checked(x_cpu, gpu, what):
    announce("quant_act_1x64", what, tuple(x_cpu.shape), x_cpu.dtype)
    q, s = bfp8.quant_act_1x64(x_cpu.to(gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x_cpu.float().numpy(), group=64)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref, err_msg=f"{what}: codes")
    np.testing.assert_array_equal(s.cpu().contiguous().numpy().view(np.uint32), s_ref.view(np.uint32),
                                  err_msg=f"{what}: scales")
    return q, s, q_ref, s_ref


def _weight(n, k, seed):
    w = workloads.weight_1x64(n, k, seed=seed)
    return w.q, w.s


@pytest.mark.parametrize("m,k,dtype", [(5, 4096, torch.float32), (7, 208, torch.bfloat16), (300, 1040, torch.float16),
                                       (1, 16, torch.bfloat16), (33, 4160, torch.bfloat16), (64, 4176, torch.float32)])
def test_quant_1x64_bit_exact(gpu, m, k, dtype):
    x = workloads.act_uniform(m, k, seed=900 + k) if dtype == torch.float32 else \
        workloads.act_normal_bf16(m, k, seed=901 + k).to(dtype)
    _quant_checked(x, gpu, f"{m}x{k}")


# K tails: 1040 = 8 x 128 + 16 (the last block's second group absent), 4160 (its second group
# absent, the first full), 4176 (first full, second 16 wide); the M values reach every K-split
# tile (16x16 to 64x64) and large M.
@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (16, 520, 1040), (40, 1000, 4160), (100, 4096, 4176),
                                   (256, 2048, 2048), (700, 520, 1024)])
def test_gemm_1x64_against_oracle(gpu, m, n, k):
    x = workloads.act_uniform(m, k, seed=910 + m)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, f"gemm {m}x{n}x{k}")
    wq, ws = _weight(n, k, 911 + n % 97)
    announce("gemm_1x64", m, n, k)
    c = bfp8.gemm_1x64(q, s, bfp8.pad_k(wq.to(gpu)), ws.to(gpu))
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 64 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 48, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, wq.numpy(), ws.numpy(), rows=rows, k_block=64)
    tolerance.compare(bits(c)[rows], ref_bits, mass, k, f"gemm_1x64 {m}x{n}x{k}", k_block=64)


def test_gemm_1x64_at_the_sweep_size_sampled(gpu):
    m, n, k = 8192, 4096, 4096
    x = workloads.act_uniform(m, k, seed=920)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, "sweep 8192")
    wq, ws = _weight(n, k, 921)
    announce("gemm_1x64 sweep size", m, n, k)
    c = bfp8.gemm_1x64(q, s, wq.to(gpu), ws.to(gpu))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(922).choice(m, 32, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, wq.numpy(), ws.numpy(), rows=rows, k_block=64)
    tolerance.compare(bits(c)[rows], ref_bits, mass, k, "gemm_1x64 8192x4096x4096", k_block=64)


def test_gemm_1x64_deterministic_and_equal_half_scales(gpu):
    """Run to run bit-equal; and with both 64-halves of every 128 columns sharing a scale the
    product is the 1x128 one to within the float32 floor (the kernels sum in different steps)."""
    m, n, k = 200, 1024, 2048
    x = workloads.act_uniform(m, k, seed=930)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, "determinism")
    wq, ws = _weight(n, k, 931)
    wq_d, ws_d = wq.to(gpu), ws.to(gpu)
    announce("gemm_1x64 determinism", m, n, k)
    a = bfp8.gemm_1x64(q, s, wq_d, ws_d)
    b = bfp8.gemm_1x64(q, s, wq_d, ws_d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # equal half scales: activation scales of the 1x128 quantizer repeated, weight scales repeated
    q128, s128 = bfp8.quant_act(x.to(gpu))
    ws128 = ws[:, 0::2].contiguous()
    s_rep = s128.t().contiguous().repeat_interleave(2, dim=0).t()  # group-major [M, 2 * K/128]
    ws_rep = ws128.repeat_interleave(2, dim=1).contiguous()
    announce("gemm_1x64 vs gemm, equal half scales", m, n, k)
    c64 = bfp8.gemm_1x64(q128, s_rep, wq_d, ws_rep.to(gpu))
    c128 = bfp8.gemm(q128, s128, wq_d, ws128.to(gpu))
    torch.cuda.synchronize()
    q128_ref, s128_ref = quant.quant_act_ref(x.numpy())
    rows = np.arange(0, m, 7)
    _, _, ref_bits, mass = tolerance.reference(q128_ref, s128_ref, wq.numpy(), ws128.numpy(), rows=rows)
    tolerance.compare(bits(c64)[rows], ref_bits, mass, k, "gemm_1x64 equal halves vs 1x128 oracle", k_block=64)
    tolerance.compare(bits(c128)[rows], ref_bits, mass, k, "gemm 1x128 (same inputs)")


# The tiled schedule (one 32x32x64 matrix-core product and one promotion per sub-tile and 64-wide
# group; 128 x 128, 256 x 128 or 256 x 256 tiles), forced on shapes the automatic choice gives the
# K-split kernel and taken by default from mid M: ragged M and N, one and several tiles per XCD,
# K tails where the last 128-wide block has a partial or absent second group (on every tile
# shape), a K of one block or less (one group, full or partial), and output rows that allow only
# 8-byte stores.
@pytest.mark.parametrize("m,n,k", [(128, 256, 1024), (300, 520, 1040), (1000, 4096, 4160), (700, 1000, 4176),
                                   (2048, 4096, 4096), (2100, 4096, 1040), (513, 384, 128), (96, 300, 208),
                                   (4100, 4096, 1040), (4096, 4004, 208), (4096, 4096, 128), (4096, 4096, 64),
                                   (4096, 4096, 16), (1000, 4096, 48)])
def test_gemm_1x64_tiled_against_oracle(gpu, m, n, k):
    x = workloads.act_uniform(m, k, seed=940 + m)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, f"tiled {m}x{n}x{k}")
    wq, ws = _weight(n, k, 941 + n % 89)
    announce("gemm_1x64 tiled", m, n, k)
    bfp8.set_schedule("tiled")
    try:
        c = bfp8.gemm_1x64(q, s, bfp8.pad_k(wq.to(gpu)), ws.to(gpu))
        c2 = bfp8.gemm_1x64(q, s, bfp8.pad_k(wq.to(gpu)), ws.to(gpu))
        torch.cuda.synchronize()
    finally:
        bfp8.set_schedule("auto")
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16)), "run to run"
    rows = np.arange(m) if m <= 128 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 64, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, wq.numpy(), ws.numpy(), rows=rows, k_block=64)
    # K below one block: a few products per group, held to the matrix core's alignment window too
    hw = tolerance.block_max_mass(q_ref, s_ref, wq.numpy(), ws.numpy(), rows, np.arange(n), 64) if k < 128 else None
    tolerance.compare(bits(c)[rows], ref_bits, mass, k, f"gemm_1x64 tiled {m}x{n}x{k}", hw_block=hw, k_block=64)


def test_gemm_1x64_schedule_choice(gpu):
    """Large M takes the tiled kernel by default; a forced K-split gives results of the same
    oracle at that size (sampled rows)."""
    m, n, k = 4096, 4096, 2048
    x = workloads.act_uniform(m, k, seed=950)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, "schedule choice")
    wq, ws = _weight(n, k, 951)
    wq_d, ws_d = wq.to(gpu), ws.to(gpu)
    announce("gemm_1x64 auto vs forced K-split", m, n, k)
    c_auto = bfp8.gemm_1x64(q, s, wq_d, ws_d)
    bfp8.set_schedule("small_m")
    try:
        c_ks = bfp8.gemm_1x64(q, s, wq_d, ws_d)
        torch.cuda.synchronize()
    finally:
        bfp8.set_schedule("auto")
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(952).choice(m, 40, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, wq.numpy(), ws.numpy(), rows=rows, k_block=64)
    tolerance.compare(bits(c_auto)[rows], ref_bits, mass, k, "gemm_1x64 auto (tiled)", k_block=64)
    tolerance.compare(bits(c_ks)[rows], ref_bits, mass, k, "gemm_1x64 forced K-split", k_block=64)


# Output rows that allow only 2-byte (ldc odd) or 8-byte (ldc % 8 == 4) stores, on each tiled
# shape (128 x 128, 256 x 128, 256 x 256); the columns past N must stay untouched.
@pytest.mark.parametrize("m", [1000, 2048, 4096])
@pytest.mark.parametrize("pad", [3, 4])
def test_gemm_1x64_tiled_padded_output(gpu, m, pad):
    n, k = 4096, 1040
    x = workloads.act_uniform(m, k, seed=960 + m)
    q, s, q_ref, s_ref = _quant_checked(x, gpu, f"padded out {m}x{n}x{k}")
    wq, ws = _weight(n, k, 961)
    buf = torch.full((m, n + pad), -7.0, dtype=torch.bfloat16, device=gpu)
    announce("gemm_1x64 padded output", m, n, k, "ldc", n + pad)
    bfp8.gemm_1x64(q, s, bfp8.pad_k(wq.to(gpu)), ws.to(gpu), out=buf[:, :n])
    torch.cuda.synchronize()
    assert (buf[:, n:] == -7.0).all(), "columns past N were written"
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m + pad).choice(m, 40, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, wq.numpy(), ws.numpy(), rows=rows, k_block=64)
    tolerance.compare(bits(buf[:, :n])[rows], ref_bits, mass, k, f"gemm_1x64 {m}x{n}x{k} ldc {n + pad}", k_block=64)
