"""GPU tests of the linear layer's one-launch path at small M, N and K, where the K-split GEMM quantizes
the bf16/fp16 activations itself: bit-identical to quantizing first (bfp8_quant_act) and then
multiplying (bfp8_gemm / bfp8_gemm_f16) with the bias added to the rounded result as the output
step adds it, for every schedule; and against the oracle's linear layer.

Inputs: the sweep's normal activations, K tails (K % 128 = 16 and 80), ragged N, strided rows,
the hidden-5120 layer shapes, and groups built to stress the quantizer's arithmetic: values
one ulp around e4m3 rounding ties, signed zeros, subnormals, the largest finite values, and
groups holding +-Inf or NaN."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import linear
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def _two_launch(x, wq, ws, bias):
    """Quantize, multiply, then add the bias to the rounded product as the output step does."""
    q, s = bfp8.quant_act(x)
    c = bfp8.gemm_f16(q, s, wq, ws) if x.dtype == torch.float16 else bfp8.gemm(q, s, wq, ws)
    if bias is not None:
        c = (c.float() + bias.float()).to(x.dtype)
    return c


def _check(x, wq, ws, bias, what, fused=True):
    m, k = x.shape
    n = wq.shape[0]
    assert bfp8.linear_fuses(m, n, k, x.stride(0)) == fused, what
    announce("linear fused", what, m, n, k, x.dtype)
    got = bfp8.linear(x, wq, ws, bias)
    want = _two_launch(x, wq, ws, bias)
    torch.cuda.synchronize()
    g, w_ = got.view(torch.int16), want.view(torch.int16)
    if not torch.equal(g, w_):
        idx = torch.nonzero(g != w_)
        raise AssertionError(f"{what}: {len(idx)} outputs differ, first at {tuple(idx[0].tolist())}")
    return got


# one, four and eight quantized rows (M = 1, 2-4, 5-8), K tails of 16 and 80, ragged N, strided
# rows; M = 16 takes the two launches (the same equality holds)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,n,k,ldx,fused", [(1, 4096, 4096, None, True), (8, 4096, 4096, None, True),
                                             (16, 4096, 4096, None, False), (7, 1000, 1040, None, True),
                                             (3, 136, 16, None, True), (1, 264, 2000, 2072, True),
                                             (6, 264, 2000, 2072, True), (5, 520, 4096, 4160, True),
                                             (2, 4096, 8192, None, True)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_fused_equals_quantize_then_gemm(gpu, dtype, m, n, k, ldx, fused, with_bias):
    w = workloads.weight(n, k, seed=800 + n % 97)
    wq, ws = bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu)
    base = workloads.act_normal_bf16(m, ldx or k, seed=801 + m).to(dtype).to(gpu)
    x = base[:, :k] if ldx else base
    bias = (torch.from_numpy(np.random.default_rng(802).standard_normal(n).astype(np.float32)).to(dtype).to(gpu)
            if with_bias else None)
    _check(x, wq, ws, bias, f"{m}x{n}x{k} ldx={ldx} {dtype} bias={with_bias}", fused=fused)


@pytest.mark.parametrize("layer", ["qkv", "o_proj", "gate_up", "down"])
@pytest.mark.parametrize("m", [1, 16])
def test_fused_on_the_hidden_5120_layers(gpu, layer, m):
    n, k = workloads.TRANSFORMER_LAYERS[layer]
    w = workloads.transformer_weight(layer)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    x = workloads.transformer_act(layer, m).to(gpu)
    _check(x, wq, ws, None, f"{layer} M={m}", fused=bfp8.linear_fuses(m, n, k))


@pytest.mark.parametrize("sched", ["auto", "small_m", "tiled"])
def test_every_schedule(gpu, sched):
    """Forced K-split and automatic: one launch; forced tiled: the two launches. Each equals
    quantize-then-GEMM under the same schedule."""
    bfp8.set_schedule(sched)
    m, n, k = 3, 2048, 3072
    w = workloads.weight(n, k, seed=810)
    bias = torch.from_numpy(np.random.default_rng(811).standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    _check(workloads.act_normal_bf16(m, k, seed=812).to(gpu), w.q.to(gpu), w.s.to(gpu), bias.to(gpu),
           f"schedule {sched}", fused=sched != "tiled")


def _tie_rows(dtype, k, seed):
    """16 rows of k values whose 1x128 groups stress the quantizer: group g of row r has amax
    448 * 2^e (a power-of-two scale, so x / s is exact) and its other values at e4m3 rounding
    ties and one ulp of the input format on either side; some groups hold signed zeros,
    subnormals, the format's largest value, +-Inf or NaN."""
    rng = np.random.default_rng(seed)
    fmt_max = 65504.0 if dtype == torch.float16 else 3.3895313892515355e38
    rows = np.zeros((16, k), np.float64)
    # e4m3 magnitudes and the midpoints between neighbours (4 significant bits: exact in bf16/fp16)
    grid = np.unique(np.concatenate([[0.0], [m * 2.0**e for e in range(-9, 9) for m in (1, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875)]]))
    grid = grid[grid <= 448]
    mids = (grid[1:] + grid[:-1]) / 2
    for r in range(16):
        for g in range(k // 128):
            e = int(rng.integers(-6, 4)) if dtype == torch.float16 else int(rng.integers(-30, 30))
            scale = 2.0**e
            vals = rng.choice(mids, 128) * scale
            kind = (r * 7 + g) % 9
            if kind == 1:
                vals[:64] = -0.0
            elif kind == 2:
                vals[:32] = rng.choice([-1, 1], 32) * (2.0**-133 if dtype == torch.bfloat16 else 2.0**-24) * rng.integers(1, 64, 32)
            vals[0] = 448 * scale
            rows[r, g * 128:(g + 1) * 128] = vals * rng.choice([-1, 1], 128)
            if kind == 3:
                rows[r, g * 128 + 5] = fmt_max
            if kind == 4 and r in (4, 13):
                rows[r, g * 128 + 9] = np.inf if r == 4 else -np.inf
            if kind == 5 and r == 5:
                rows[r, g * 128 + 17] = np.nan
    x = torch.from_numpy(rows.astype(np.float32)).to(dtype)
    # one ulp of the input format on either side of the ties
    bits16 = x.view(torch.int16).clone()
    flip = torch.from_numpy(rng.integers(-1, 2, bits16.shape)).to(torch.int16)
    fin = torch.isfinite(x)
    finite = fin & (x != 0) & (x.abs() < x.abs()[fin].max())
    bits16[finite] += flip[finite]
    return bits16.view(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fused_quantizer_arithmetic_on_ties_and_special_values(gpu, dtype):
    n, k = 256, 1024
    w = workloads.weight(n, k, seed=820)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    x = _tie_rows(dtype, k, 821).to(gpu)
    for m in (8, 5, 4, 1):
        _check(x[:m].contiguous(), wq, ws, None, f"ties/special M={m}")
    for m in (16,):  # the two launches: the quantizer alone on the same rows
        _check(x[:m].contiguous(), wq, ws, None, f"ties/special M={m}", fused=False)


def test_fused_against_the_oracle(gpu):
    """The one-launch layer against the oracle's linear layer (quantize, blockwise product,
    bf16 rounding, bias), under the GEMM's bound plus one bf16 ulp of the output."""
    m, n, k = 4, 1000, 2176
    w = workloads.weight(n, k, seed=830)
    x = workloads.act_normal_bf16(m, k, seed=831)
    bias = torch.from_numpy(np.random.default_rng(832).standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy())
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
    assert bfp8.linear_fuses(m, n, k)
    announce("linear fused vs oracle", m, n, k)
    got = bfp8.linear(x.to(gpu), w.q.to(gpu), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    tolerance.compare_linear(bits(got), out_ref, c_ref, mag, k, "linear fused vs oracle")


def test_noalloc_takes_the_same_path(gpu):
    m, n, k = 4, 512, 1536
    w = workloads.weight(n, k, seed=840)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    x = workloads.act_normal_bf16(m, k, seed=841).to(gpu)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=gpu)
    announce("linear_noalloc fused", m, n, k)
    bfp8.linear_noalloc(x, wq, ws, out)
    want = _two_launch(x, wq, ws, None)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
