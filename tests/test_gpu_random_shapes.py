"""GPU parity over seeded random shapes: the automatic schedule and tile choices (K-split or tiled;
the tiled plans with their column splits and fewest-round shapes; the 1x64 kernel's three tile
shapes; the UE8M0 and fp16-output forms; the linear layer's one-launch or two-launch path; the
grouped GEMM over random expert counts) on ragged M, N and K, each against the oracle on sampled
rows, with output rows padded (or padding rows preset) so that what must stay untouched can be
checked."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import f16, gemm, linear, quant, ue8m0
from tests import tolerance
from tests.gpu_util import announce, bits, quant_gpu_checked

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


def _linear_shapes(count):
    out = []
    for _ in range(count):
        m = int(_RNG.choice([_RNG.integers(1, 9), _RNG.integers(9, 300), _RNG.integers(300, 2500)]))
        out.append((m, int(_RNG.integers(1, 3000)), int(_RNG.integers(8, 262)) * 16))
    return out


def _grouped_shapes(count):
    return [(int(_RNG.integers(1, 13)), int(_RNG.integers(1, 2500)), int(_RNG.integers(1, 2049)),
             int(_RNG.integers(8, 129)) * 16) for _ in range(count)]


SHAPES_LINEAR = _linear_shapes(9)
SHAPES_GROUPED = _grouped_shapes(6)


@pytest.mark.parametrize("m,n,k", SHAPES_LINEAR)
def test_linear_random_shape(gpu, m, n, k):
    """bf16 activations and a bias: the one-launch path at small M where it pays, else the
    quantizer and the GEMM."""
    w = workloads.weight(n, k, seed=n * 13 + k)
    x = workloads.act_normal_bf16(m, k, seed=m * 17 + k)
    rng = np.random.default_rng(m + n + k)
    bias = torch.from_numpy((rng.choice([-1.0, 1.0], n) * np.exp2(rng.uniform(-6, 3, n))).astype(np.float32))
    bias = bias.to(torch.bfloat16)
    rows = _rows(m, m * n + k)
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy(),
                                             rows=rows)
    mass = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), rows, np.arange(n))
    announce("linear random shape", m, n, k, "fused" if bfp8.linear_fuses(m, n, k) else "two launches")
    got = bfp8.linear(x.to(gpu), bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    tolerance.compare_linear(bits(got)[rows], out_ref, c_ref, mass, k, f"linear random {m}x{n}x{k}")


@pytest.mark.parametrize("groups,tokens,n,k", SHAPES_GROUPED)
def test_grouped_random_shape(gpu, groups, tokens, n, k):
    """Random expert counts (some experts empty), 128-row padding; padding rows stay untouched."""
    counts = workloads.moe_counts(groups, tokens, seed=groups * 31 + tokens)
    layout = workloads.moe_layout(counts)
    x = workloads.act_normal_bf16(layout.size, k, seed=tokens + k)
    x[torch.from_numpy(layout < 0)] = 0
    weights = [workloads.weight(n, k, seed=n * 7 + k + g) for g in range(groups)]
    bq = torch.stack([w.q for w in weights])
    bs = torch.stack([w.s for w in weights])
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, f"grouped random {groups}x{tokens}x{n}x{k}")
    out = torch.full((layout.size, n), 1536.0, dtype=torch.bfloat16, device=gpu)
    announce("grouped random shape", groups, tokens, layout.size, n, k)
    bfp8.grouped_gemm_contiguous(q, s, bfp8.pad_k(bq.to(gpu)), bs.to(gpu), torch.from_numpy(layout).to(gpu), out=out)
    torch.cuda.synchronize()
    assert (out[torch.from_numpy(layout < 0).to(gpu)].float() == 1536.0).all(), "padding rows were written"
    cb = bits(out)
    rng = np.random.default_rng(groups + n)
    cols = np.arange(n) if n <= 512 else np.unique(np.concatenate([[0, n - 1], rng.choice(n, 400, replace=False)]))
    for g in np.unique(layout[layout >= 0]):
        rows = np.nonzero(layout == g)[0]
        rows = np.unique(np.concatenate([rows[:1], rows[-1:], rng.choice(rows, min(4, rows.size), replace=False)]))
        _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, bq[g].numpy(), bs[g].numpy(), rows=rows, cols=cols)
        tolerance.compare(cb[np.ix_(rows, cols)], ref_bits, mass, k, f"grouped random expert {g} ({n}x{k})")


SHAPES_E8 = [(int(_RNG.choice([_RNG.integers(1, 257), _RNG.integers(257, 4300)])), int(_RNG.integers(1, 4300)),
              int(_RNG.integers(1, 33)) * 128) for _ in range(6)]
SHAPES_F16 = _shapes(6)


@pytest.mark.parametrize("m,n,k", SHAPES_E8)
def test_gemm_ue8m0_random_shape(gpu, m, n, k):
    """UE8M0 scales applied by the hardware-scaled MFMA (K a multiple of 128)."""
    x = workloads.act_normal_bf16(m, k, seed=m * 19 + k)
    q, e = bfp8.quant_act_ue8m0(x.to(gpu))
    q_ref, e_ref = ue8m0.quant_act_ue8m0_ref(x.float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(e.cpu().contiguous().numpy(), e_ref)
    w = workloads.weight_ue8m0(n, k, seed=n * 23 + k)
    buf, out = _padded_out(m, n, gpu)
    announce("gemm_ue8m0 random shape", m, n, k, "->", bfp8.schedule_for(m, n, k))
    bfp8.gemm_ue8m0(q, e, w.q.to(gpu), bfp8.ue8m0_scales(w.s.to(gpu)), out=out)
    torch.cuda.synchronize()
    assert (buf[:, n:] == -3.0).all(), "columns past N were written"
    rows = _rows(m, m + n * 3 + k)
    _, _, ref_bits, mass = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    tolerance.compare_e8(bits(out)[rows], ref_bits, mass, k, f"gemm_ue8m0 random {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", SHAPES_F16)
def test_gemm_f16_random_shape(gpu, m, n, k):
    """fp16 output."""
    x = workloads.act_normal_bf16(m, k, seed=m * 29 + k)
    q, s = bfp8.quant_act(x.to(gpu))
    q_ref, s_ref = quant.quant_act_ref(x.float().numpy())
    w = workloads.weight(n, k, seed=n * 37 + k)
    buf = torch.full((m, n + 5), -3.0, dtype=torch.float16, device=gpu)
    announce("gemm_f16 random shape", m, n, k, "->", bfp8.schedule_for(m, n, k))
    bfp8.gemm_f16(q, s, bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu), out=buf[:, :n])
    torch.cuda.synchronize()
    assert (buf[:, n:] == -3.0).all(), "columns past N were written"
    rows = _rows(m, m + n * 5 + k)
    acc, _ = gemm.gemm_acc_ref(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    mass = tolerance.masses(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, np.arange(n))
    got = buf[:, :n].detach().cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    tolerance.compare_f16(got, f16.to_bits(acc), mass, k, f"gemm_f16 random {m}x{n}x{k}")


def _moe_shapes(count):
    return [(int(_RNG.integers(1, 300)), int(_RNG.integers(1, 9)), int(_RNG.integers(1, 25)),
             int(_RNG.integers(1, 5)) * 128, int(_RNG.integers(1, 5)) * 128, float(_RNG.choice([0.0, 0.1])))
            for _ in range(count)]


SHAPES_MOE = _moe_shapes(6)


@pytest.mark.parametrize("t,top_k,e,h,i,sent", SHAPES_MOE)
def test_moe_forward_random_shape(gpu, t, top_k, e, h, i, sent):
    """The experts forward (dispatch, tokens quantized once, grouped up projection, SwiGLU +
    quantization, grouped down projection, weighted combine) on random routing (top_k drawn up to
    8 and clipped to the expert count; with sentinels for experts held elsewhere) against the
    oracle's forward, with the end-to-end bound of the benchmark-size test: 2^-2 of the down
    product's absolute mass plus 2 bf16 ulp per element, mean relative error within 2e-3 (the
    second quantization re-decides codes from up-projection outputs that differ by rounding)."""
    from tests.test_gpu_moe import _check_forward, _down_mass
    from oracle import moe

    top_k = min(top_k, e)
    x = workloads.act_normal_bf16(t, h, seed=t * 41 + h)
    ids, w = workloads.moe_routing(t, top_k, e, seed=t + e + i, sentinel_frac=sent)
    wts = workloads.moe_experts(e, h, i, seed=e * 43 + i)
    announce("moe_forward random shape", t, top_k, e, h, i, sent)
    y = bfp8.moe_forward(x.to(gpu), ids.to(gpu), w.to(gpu), *(a.to(gpu) for a in wts))
    torch.cuda.synchronize()
    ref = moe.moe_forward_ref(x.float().numpy(), ids.numpy(), w.numpy(), *(a.numpy() for a in wts))
    _check_forward(bits(y), ref, _down_mass(x, ids, w, wts), f"moe random {t}x{top_k}of{e} h{h} i{i}",
                   mean_bound=2e-3)
