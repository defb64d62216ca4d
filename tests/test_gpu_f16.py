"""GPU parity of the fp16 forms: the quantizer on fp16 activations (bit-exact), the GEMM with an fp16
output and the fp16 linear layer (output and bias in the activations' dtype) against the oracle."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import f16, gemm, linear, quant
from tests import tolerance
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


@pytest.mark.parametrize("m,k", [(1, 512), (77, 1024), (300, 7168)])
def test_quant_fp16_input(gpu, m, k):
    x = (workloads.act_normal_bf16(m, k, seed=500 + m).float() * 30).to(torch.float16)
    x[0, :128] *= 2.0**-20  # fp16 subnormals
    announce("quant_act fp16", m, k)
    q, s = bfp8.quant_act(x.to(gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x.float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().contiguous().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("m", [1, 24, 200, 600, 2048])
@pytest.mark.parametrize("sched", ["auto", "small_m", "tiled"])
def test_gemm_f16_output(gpu, m, sched):
    n, k = 1032, 1536
    w = workloads.weight(n, k, seed=510)
    x = workloads.act_normal_bf16(m, k, seed=511 + m)
    q, s = bfp8.quant_act(x.to(gpu))
    bfp8.set_schedule(sched)
    announce("gemm_f16", m, n, k, sched)
    c = bfp8.gemm_f16(q, s, w.q.to(gpu), w.s.to(gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x.float().numpy())
    rows = np.arange(m) if m <= 64 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 40, replace=False)]))
    acc, _ = gemm.gemm_acc_ref(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    mag = tolerance.masses(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, np.arange(n))
    tolerance.compare_f16(_bits16(c)[rows], f16.to_bits(acc), mag, k, f"gemm_f16 M={m} {sched}")


@pytest.mark.parametrize("m", [3, 150, 700])
@pytest.mark.parametrize("strided_out", [False, True])
def test_linear_fp16_bias_bit_exact(gpu, m, strided_out):
    """Inputs whose C is exact on every path (one nonzero product per output, power-of-two scales):
    the fp16 bias step fp16(float(fp16(C)) + float(bias)) must match bit for bit."""
    n, k = 136, 256
    rng = np.random.default_rng(600 + m)
    codes = rng.integers(0, 0x7F, (m, k)).astype(np.uint8)
    from oracle import e4m3

    vals = e4m3.decode(codes)
    for g in range(k // 128):
        vals[np.arange(m), g * 128 + rng.integers(0, 128, m)] = rng.choice([-448.0, 448.0], m)
    x = torch.from_numpy((vals * 2.0**-6).astype(np.float32)).to(torch.float16)
    w_q = np.zeros((n, k), np.uint8)
    w_q[np.arange(n), rng.integers(0, k, n)] = rng.integers(1, 0x7F, n).astype(np.uint8)
    w_s = np.exp2(rng.integers(-8, -3, (2, 2))).astype(np.float32)
    bias = torch.from_numpy(rng.uniform(-1, 1, n) * np.exp2(rng.integers(-12, 6, n))).to(torch.float16)
    out_ref, c_ref, _, _ = linear.linear_f16_ref(x.float().numpy(), w_q, w_s, bias=bias.float().numpy())
    announce("linear fp16 exact", m, strided_out)
    out = torch.empty((m, n + 3), dtype=torch.float16, device=gpu)[:, :n] if strided_out else None
    got = bfp8.linear(x.to(gpu), torch.from_numpy(w_q).to(gpu), torch.from_numpy(w_s).to(gpu), bias.to(gpu), out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits16(got), out_ref)
    got = bfp8.linear(x.to(gpu), torch.from_numpy(w_q).to(gpu), torch.from_numpy(w_s).to(gpu), None, out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits16(got), c_ref)


def test_linear_fp16_transformer_shape(gpu):
    """o_proj shapes (N = 5120, K = 8192) at M = 16 with fp16 N(0,1) activations and a bias."""
    m, n, k = 16, 5120, 8192
    w = workloads.transformer_weight("o_proj")
    x = workloads.act_normal_bf16(m, k, seed=520).to(torch.float16)
    bias = torch.from_numpy(np.random.default_rng(521).standard_normal(n)).to(torch.float16)
    announce("linear fp16 o_proj", m)
    got = bfp8.linear(x.to(gpu), w.q.to(gpu), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    out_ref, c_ref, q, s = linear.linear_f16_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy())
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
    tolerance.compare_linear(_bits16(got), out_ref, c_ref, mag, k, "linear fp16 o_proj", fmt=f16)
