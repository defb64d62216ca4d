"""GPU parity of bfp8_linear (bf16 activations -> quantize -> blockwise FP8 GEMM -> bf16 + bias)
against the oracle's linear layer.

The bias step is checked bit for bit on inputs whose GEMM result is exact (one nonzero
product per output, power-of-two scales), so that C is the same on both sides whatever the
accumulation order; the rest is checked under the GEMM's bound plus one bf16 ulp of the output."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import bf16, e4m3, linear
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def _bf16_spread(rng, shape, lo, hi):
    """bf16 values (as a float32 torch tensor) with random sign and magnitudes 2**U(lo, hi)."""
    v = rng.choice([-1.0, 1.0], shape) * np.exp2(rng.uniform(lo, hi, shape))
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)


def _exact_case(m, n, k, seed):
    """Activations, one-hot FP8 weight and power-of-two block scales for which C is exact.

    Each 128-group of a row holds one element of magnitude 448 * 2**-6, so its scale is 2**-6
    exactly and every element (e4m3 value * 2**-6) quantizes to its code without rounding.
    Each weight row has a single nonzero code; a product of two e4m3 values has at most
    8 significant bits, so C = x * w * 2**-6 * ws is a bf16 value on every path."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, (m, k)).astype(np.uint8) | (rng.integers(0, 2, (m, k)).astype(np.uint8) << 7)
    vals = e4m3.decode(codes)
    for g in range(k // 128):
        vals[np.arange(m), g * 128 + rng.integers(0, 128, m)] = rng.choice([-448.0, 448.0], m)
    x = torch.from_numpy((vals * 2.0**-6).astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(x.float(), torch.from_numpy((vals * 2.0**-6).astype(np.float32)))
    w_q = np.zeros((n, k), np.uint8)
    w_q[np.arange(n), rng.integers(0, k, n)] = rng.integers(1, 0x7F, n).astype(np.uint8) | 0x80 * rng.integers(0, 2, n).astype(np.uint8)
    w_s = np.exp2(rng.integers(-8, -1, (-(-n // 128), k // 128))).astype(np.float32)
    return x, torch.from_numpy(w_q), torch.from_numpy(w_s)


@pytest.mark.parametrize("m", [1, 37, 128, 300])
@pytest.mark.parametrize("sched", ["auto", "small_m", "tiled"])
@pytest.mark.parametrize("strided_out", [False, True])
def test_bias_epilogue_bit_exact(gpu, m, sched, strided_out):
    """Bias added in the kernels' bf16 output step equals bf16(float32(bf16(C)) + bias) bit for
    bit, for the staged (row stride a multiple of 8) and the direct (odd row stride) stores."""
    n, k = 136, 256
    x, w_q, w_s = _exact_case(m, n, k, seed=m)
    rng = np.random.default_rng(1000 + m)
    bias = _bf16_spread(rng, (n,), -30, 12)
    _, c_ref, _, _ = linear.linear_ref(x.float().numpy(), w_q.numpy(), w_s.numpy())
    c_val = bf16.from_bits(c_ref)
    bias[:8] = torch.from_numpy(-c_val[0, :8].astype(np.float32)).to(torch.bfloat16)  # exact cancellation
    bias[8:16] = torch.from_numpy(c_val[0, 8:16].astype(np.float32) * 2.0**-9).to(torch.bfloat16)  # rounding ties region
    out_ref, _, _, _ = linear.linear_ref(x.float().numpy(), w_q.numpy(), w_s.numpy(), bias=bias.float().numpy())
    bfp8.set_schedule(sched)
    announce("linear exact", m, n, k, sched, "strided" if strided_out else "dense")
    out = torch.empty((m, n + 3), dtype=torch.bfloat16, device=gpu)[:, :n] if strided_out else None
    got = bfp8.linear(x.to(gpu), w_q.to(gpu), w_s.to(gpu), bias.to(gpu), out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(got), out_ref)
    announce("linear exact no bias", m, sched)
    got = bfp8.linear(x.to(gpu), w_q.to(gpu), w_s.to(gpu), None, out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(got), c_ref)


def test_page2_shapes_with_bias(gpu):
    """83 x 576 x 7168 (the page's test shapes) with N(0,1) bf16 activations and a bias."""
    m, n, k = 83, 576, 7168
    w = workloads.weight(n, k, seed=5)
    x = workloads.act_normal_bf16(m, k, seed=6)
    bias = _bf16_spread(np.random.default_rng(7), (n,), -4, 2)
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy())
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
    announce("linear page2 shapes", m, n, k)
    got = bfp8.linear(x.to(gpu), w.q.to(gpu), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    print(tolerance.compare_linear(bits(got), out_ref, c_ref, mag, k, "linear page2"))


_square = {}


@pytest.mark.parametrize("m", [1, 9, 128, 300, 1024])
def test_square_with_bias_sampled_rows(gpu, m):
    n = k = 4096
    if "w" not in _square:
        w = workloads.weight(n, k, seed=8)
        _square["w"] = (w, w.q.to(gpu), w.s.to(gpu))
    w, wq, ws = _square["w"]
    x = workloads.act_normal_bf16(m, k, seed=50 + m)
    bias = _bf16_spread(np.random.default_rng(m), (n,), -6, 3)
    rows = np.arange(m) if m <= 16 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 14, replace=False)]))
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy(), rows=rows)
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), rows, np.arange(n))
    announce("linear square", m, n, k, "->", bfp8.schedule_for(m, n, k))
    got = bfp8.linear(x.to(gpu), wq, ws, bias.to(gpu))
    torch.cuda.synchronize()
    print(tolerance.compare_linear(bits(got)[rows], out_ref, c_ref, mag, k, f"linear square M={m}"))


@pytest.mark.parametrize("m", [64, 128])
def test_wide_gate_up_weight_sampled_rows(gpu, m):
    """The hidden-5120 gate+up projection (N = 51200, K = 5120), where the automatic choice
    takes the tiled schedule below 256 rows; sampled rows against the oracle."""
    n, k = 51200, 5120
    if "wide" not in _square:
        w = workloads.weight(n, k, seed=12)
        _square["wide"] = (w, w.q.to(gpu), w.s.to(gpu))
    w, wq, ws = _square["wide"]
    assert bfp8.schedule_for(m, n, k) == "tiled"
    x = workloads.act_normal_bf16(m, k, seed=80 + m)
    bias = _bf16_spread(np.random.default_rng(m + 1), (n,), -6, 3)
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 6, replace=False)]))
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy(), rows=rows)
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), rows, np.arange(n))
    announce("linear wide", m, n, k, "->", bfp8.schedule_for(m, n, k))
    got = bfp8.linear(x.to(gpu), wq, ws, bias.to(gpu))
    torch.cuda.synchronize()
    print(tolerance.compare_linear(bits(got)[rows], out_ref, c_ref, mag, k, f"linear wide M={m}"))


def test_without_bias_equals_quantize_then_gemm(gpu):
    """The fused layer is the two entry points back to back: same bits, both schedules."""
    n, k = 1000, 1536
    w = workloads.weight(n, k, seed=9)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    for m, sched in [(5, "small_m"), (200, "small_m"), (200, "tiled"), (700, "tiled")]:
        bfp8.set_schedule(sched)
        x = workloads.act_normal_bf16(m, k, seed=60 + m).to(gpu)
        announce("linear vs quant+gemm", m, n, k, sched)
        got = bfp8.linear(x, wq, ws)
        q, s = bfp8.quant_act(x)
        want = bfp8.gemm(q, s, wq, ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (m, sched)


def test_caller_workspace_back_to_back(gpu):
    """A caller-owned workspace sized for the largest call, reused by smaller ones, and rows of
    x with a stride larger than K."""
    n, k = 264, 640
    w = workloads.weight(n, k, seed=10)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    bias = _bf16_spread(np.random.default_rng(3), (n,), -3, 3)
    sizes = [512, 3, 260, 64, 1]
    nbytes = max(bfp8.linear_workspace_bytes(m, n, k) for m in sizes)
    work = torch.empty(nbytes, dtype=torch.uint8, device=gpu)
    for m in sizes:
        xs = workloads.act_normal_bf16(m, k + 72, seed=70 + m)
        x = xs[:, :k]
        out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy())
        mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
        announce("linear caller workspace", m, n, k)
        got = bfp8.linear(xs.to(gpu)[:, :k], wq, ws, bias.to(gpu), workspace=work)
        torch.cuda.synchronize()
        tolerance.compare_linear(bits(got), out_ref, c_ref, mag, k, f"linear workspace M={m}")


def test_empty_batch(gpu):
    w = workloads.weight(128, 256, seed=11)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=gpu)
    out = bfp8.linear(x, w.q.to(gpu), w.s.to(gpu), torch.zeros(128, dtype=torch.bfloat16, device=gpu))
    assert out.shape == (0, 128)
