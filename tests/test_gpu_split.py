"""GPU parity of GEMMs whose tiles fill the chip a whole number of times plus a fraction: the
tiled schedule then runs the columns of that fraction as a second launch with smaller tiles.
Both column ranges are checked against the oracle for every output form (bf16 and fp16 C,
UE8M0 scales, the linear layer's bias, a partial last K block) and with padded strides."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import f16, gemm, linear, ue8m0
from tests import tolerance
from tests.gpu_util import announce, bits, quant_gpu_checked

pytestmark = pytest.mark.gpu

# (M, N, K): 320 tiles of 256 x 256 (qkv-like) and of 256 x 128 (o_proj-like), 800 of 256 x 256
SPLIT_SHAPES = [(2048, 10240, 1024), (2048, 5120, 2048), (1024, 51200, 512)]


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def _rows_cols(m, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 22, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(256), np.arange(n - 1300, n), rng.choice(n, 600, replace=False)]))
    return rows, cols


@pytest.mark.parametrize("m,n,k", SPLIT_SHAPES)
def test_split_gemm_bf16_and_strided_out(gpu, m, n, k):
    w = workloads.weight(n, k, seed=n)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.act_uniform(m, k, seed=m), gpu, f"split {m}x{n}x{k}")
    bfp8.set_schedule("tiled")
    announce("gemm split", m, n, k)
    out = torch.full((m, n + 8), -1.0, dtype=torch.bfloat16, device=gpu)
    c = bfp8.gemm(q, s, w.q.to(gpu), w.s.to(gpu), out=out[:, :n])
    torch.cuda.synchronize()
    rows, cols = _rows_cols(m, n, seed=k)
    _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows, cols=cols)
    tolerance.compare(bits(c)[np.ix_(rows, cols)], ref_bits, mag, k, f"split {m}x{n}x{k}")
    assert (out[:, n:].float() == -1.0).all()


def test_split_gemm_f16(gpu):
    m, n, k = SPLIT_SHAPES[0]
    w = workloads.weight(n, k, seed=3)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.act_normal_bf16(m, k, seed=4), gpu, "split f16")
    announce("gemm_f16 split", m, n, k)
    c = bfp8.gemm_f16(q, s, w.q.to(gpu), w.s.to(gpu))
    torch.cuda.synchronize()
    rows, cols = _rows_cols(m, n, seed=5)
    acc, _ = gemm.gemm_acc_ref(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows, cols=cols)
    mag = tolerance.masses(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, cols)
    got = c.cpu().view(torch.int16).numpy().view(np.uint16)[np.ix_(rows, cols)]
    tolerance.compare_f16(got, f16.to_bits(acc), mag, k, "split f16")


def test_split_gemm_ue8m0(gpu):
    m, n, k = SPLIT_SHAPES[1]
    a = workloads.act_uniform(m, k, seed=6)
    announce("quant_act_ue8m0 split", m, k)
    q, e = bfp8.quant_act_ue8m0(a.to(gpu))
    torch.cuda.synchronize()
    q_ref, e_ref = ue8m0.quant_act_ue8m0_ref(a.numpy())
    assert np.array_equal(q.cpu().numpy(), q_ref)
    w = workloads.weight_ue8m0(n, k, seed=7)
    announce("gemm_ue8m0 split", m, n, k)
    c = bfp8.gemm_ue8m0(q, e, w.q.to(gpu), bfp8.ue8m0_scales(w.s.to(gpu)))
    torch.cuda.synchronize()
    rows, cols = _rows_cols(m, n, seed=8)
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy(), rows=rows, cols=cols)
    tolerance.compare_e8(bits(c)[np.ix_(rows, cols)], ref_bits, mag, k, "split ue8m0")


def test_split_linear_with_bias(gpu):
    m, n, k = SPLIT_SHAPES[0]
    x = workloads.act_normal_bf16(m, k, seed=9)
    w = workloads.weight(n, k, seed=10)
    bias = torch.from_numpy(np.random.default_rng(11).standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    announce("linear split", m, n, k)
    y = bfp8.linear(x.to(gpu), w.q.to(gpu), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    rows, cols = _rows_cols(m, n, seed=12)
    out_ref, c_ref, q, s = linear.linear_ref(x[rows].float().numpy(), w.q.numpy(), w.s.numpy(),
                                             bias=bias.float().numpy(), cols=cols)
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(rows.size), cols)
    tolerance.compare_linear(bits(y)[np.ix_(rows, cols)], out_ref, c_ref, mag, k, "split linear")


def test_split_partial_last_k_block(gpu):
    m, n, k = 2048, 10240, 1008
    w = workloads.weight(n, k, seed=13)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.act_uniform(m, k, seed=14), gpu, "split ktail")
    announce("gemm split ktail", m, n, k)
    c = bfp8.gemm(q, s, bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu))
    torch.cuda.synchronize()
    rows, cols = _rows_cols(m, n, seed=15)
    _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows, cols=cols)
    tolerance.compare(bits(c)[np.ix_(rows, cols)], ref_bits, mag, k, "split ktail")
