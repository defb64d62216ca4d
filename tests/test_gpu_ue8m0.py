"""GPU parity of the UE8M0 (power-of-two scale) entry points against the oracle: the quantizer
bit for bit, the dense and grouped GEMMs under the bound of the hardware-scaled accumulation."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import ue8m0
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu

SCHEDULES = ["auto", "small_m", "tiled"]


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def quant_e8_checked(x_cpu, dev, what=""):
    """GPU UE8M0 quantization, asserted bit-exact against the oracle; returns device and host results."""
    announce("quant_act_ue8m0", what, tuple(x_cpu.shape), x_cpu.dtype)
    q, e = bfp8.quant_act_ue8m0(x_cpu.to(dev))
    torch.cuda.synchronize()
    q_ref, e_ref = ue8m0.quant_act_ue8m0_ref(x_cpu.float().numpy())
    q_got, e_got = q.cpu().numpy(), e.cpu().contiguous().numpy()
    if not np.array_equal(q_got, q_ref):
        i = tuple(np.argwhere(q_got != q_ref)[0])
        raise AssertionError(f"{what}: codes differ at {i}: got {q_got[i]:#x} want {q_ref[i]:#x}")
    if not np.array_equal(e_got, e_ref):
        i = tuple(np.argwhere(e_got != e_ref)[0])
        raise AssertionError(f"{what}: scale codes differ at {i}: got {e_got[i]} want {e_ref[i]}")
    return q, e, q_ref, e_ref


@pytest.mark.parametrize("m", [1, 37, 300, 4096])  # 4096 x 8 groups: the 8-lanes-per-group mapping
def test_quant_fp32_uniform(gpu, m):
    quant_e8_checked(workloads.act_uniform(m, 1024, seed=400 + m), gpu, f"uniform M={m}")


def test_quant_bf16_zero_groups_and_wide_range(gpu):
    x = workloads.act_normal_bf16(130, 640, seed=401)
    x[3, 128:256] = 0
    x[5] *= 2.0**40
    x[6] *= 2.0**-60
    quant_e8_checked(x, gpu, "bf16 zero groups, wide range")


def test_quant_strided_rows_and_padded_scales(gpu):
    xs = workloads.act_uniform(45, 512 + 32, seed=402)
    announce("quant_act_ue8m0 strided", 45)
    x = xs.to(gpu)[:, :512]
    scales = torch.full((4, 52), 0xAA, dtype=torch.uint8, device=gpu)[:, :45].t()
    q, e = bfp8.quant_act_ue8m0(x, scales=scales)
    torch.cuda.synchronize()
    q_ref, e_ref = ue8m0.quant_act_ue8m0_ref(xs[:, :512].numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(e.cpu().numpy(), e_ref)
    # the padding of the scale rows is not written
    pad = torch.as_strided(e, (4, 7), (52, 1), e.storage_offset() + 45)
    assert (pad == 0xAA).all()


def _weight_e8(dev, n, k, seed):
    w = workloads.weight_ue8m0(n, k, seed)
    return w, w.q.to(dev), bfp8.ue8m0_scales(w.s.to(dev))


def _gemm_e8(sched, q, e, bq, be, what, out=None):
    bfp8.set_schedule(sched)
    announce("gemm_ue8m0", what, sched, "->", bfp8.schedule_for(q.shape[0], bq.shape[0], q.shape[1]))
    c = bfp8.gemm_ue8m0(q, e, bq, be, out=out)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("sched", SCHEDULES)
def test_page2_shapes(gpu, sched):
    """83 x 576 x 7168 with U(-448, 448) activations (the page's test shapes), UE8M0 scales."""
    w, bq, be = _weight_e8(gpu, 576, 7168, seed=410)
    q, e, q_ref, e_ref = quant_e8_checked(workloads.act_uniform(83, 7168, seed=411), gpu, "page2 shapes")
    c = _gemm_e8(sched, q, e, bq, be, "page2 83x576x7168")
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy())
    print(sched, tolerance.compare_e8(bits(c), ref_bits, mag, 7168, f"page2 e8 {sched}"))


_sq = {}


@pytest.mark.parametrize("m", [1, 9, 16, 64, 128, 256, 512, 2048, 8192])
def test_square_sweep(gpu, m):
    if "w" not in _sq:
        _sq["w"] = _weight_e8(gpu, 4096, 4096, seed=412)
    w, bq, be = _sq["w"]
    q, e, q_ref, e_ref = quant_e8_checked(workloads.square_act(m), gpu, f"square M={m}")
    c = _gemm_e8("auto", q, e, bq, be, f"square M={m}")
    rows = np.arange(m) if m <= 16 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 30, replace=False)]))
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    print(m, tolerance.compare_e8(bits(c)[rows], ref_bits, mag, 4096, f"square e8 M={m}"))


@pytest.mark.parametrize("m,n,k", [(5, 136, 384), (130, 264, 640), (600, 392, 256)])
@pytest.mark.parametrize("sched", ["small_m", "tiled"])
def test_ragged_tails(gpu, m, n, k, sched):
    w, bq, be = _weight_e8(gpu, n, k, seed=413 + m)
    q, e, q_ref, e_ref = quant_e8_checked(workloads.act_normal_bf16(m, k, seed=414 + m), gpu, f"ragged {m}x{n}x{k}")
    out = torch.full((m, n + 5), 7.0, dtype=torch.bfloat16, device=gpu)[:, :n]
    c = _gemm_e8(sched, q, e, bq, be, f"ragged {m}x{n}x{k}", out=out)
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy())
    tolerance.compare_e8(bits(c), ref_bits, mag, k, f"ragged e8 {m}x{n}x{k} {sched}")
    assert (torch.as_strided(out, (m, 5), (n + 5, 1), n).float().cpu() == 7.0).all()


def test_agrees_with_float_scale_path(gpu):
    """The same power-of-two scales through bfp8_gemm (float scales, VALU promotion) and through
    bfp8_gemm_ue8m0 (hardware-scaled accumulation): both near the oracle, and near each other."""
    m, n, k = 1024, 1024, 2048
    w, bq, be = _weight_e8(gpu, n, k, seed=415)
    q, e, q_ref, e_ref = quant_e8_checked(workloads.act_normal_bf16(m, k, seed=416), gpu, "float vs e8")
    s_f = torch.from_numpy(ue8m0.decode(e.cpu().numpy()).astype(np.float32)).to(gpu)
    s_f = s_f.t().contiguous().t()  # group-major float scales
    bs_f = torch.from_numpy(ue8m0.decode(w.s.numpy()).astype(np.float32)).to(gpu)
    announce("gemm float-scale vs ue8m0", m, n, k)
    c_f = bfp8.gemm(q, s_f, bq, bs_f)
    c_e = bfp8.gemm_ue8m0(q, e, bq, be)
    torch.cuda.synchronize()
    rows = np.arange(0, m, 37)
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    tolerance.compare(bits(c_f)[rows], ref_bits, mag, k, "float-scale path")
    tolerance.compare_e8(bits(c_e)[rows], ref_bits, mag, k, "ue8m0 path")
    d = (c_f.float() - c_e.float()).abs().mean() / c_f.float().abs().mean()
    assert d.item() < 1e-3


@pytest.mark.parametrize("m", [16, 2048])
def test_run_to_run_bitwise(gpu, m):
    if "w" not in _sq:
        _sq["w"] = _weight_e8(gpu, 4096, 4096, seed=412)
    w, bq, be = _sq["w"]
    q, e = bfp8.quant_act_ue8m0(workloads.square_act(m).to(gpu))
    announce("gemm_ue8m0 determinism", m)
    c0 = bfp8.gemm_ue8m0(q, e, bq, be)
    c1 = bfp8.gemm_ue8m0(q, e, bq, be)
    torch.cuda.synchronize()
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))


def test_grouped_moe_layout(gpu):
    """4 experts, N=512, K=1024, Dirichlet token counts, 128-row padding; UE8M0 scales."""
    counts = workloads.moe_counts(groups=4, tokens=700, seed=420)
    layout = workloads.moe_layout(counts)
    ws = [workloads.weight_ue8m0(512, 1024, seed=421 + g) for g in range(4)]
    bq = torch.stack([w.q for w in ws])
    be = torch.stack([w.s for w in ws])
    x = workloads.act_normal_bf16(layout.size, 1024, seed=425)
    x[torch.from_numpy(layout < 0)] = 0
    q, e, q_ref, e_ref = quant_e8_checked(x, gpu, "grouped activations")
    lay_d = torch.from_numpy(layout).to(gpu)
    out = torch.full((layout.size, 512), 1536.0, dtype=torch.bfloat16, device=gpu)
    announce("grouped_gemm_ue8m0", layout.size)
    c = bfp8.grouped_gemm_contiguous_ue8m0(q, e, bq.to(gpu), bfp8.ue8m0_scales(be.to(gpu)), lay_d, out=out)
    torch.cuda.synchronize()
    cb = bits(c)
    for g in range(4):
        rows = np.nonzero(layout == g)[0]
        if rows.size == 0:
            continue
        _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, bq[g].numpy(), be[g].numpy(), rows=rows)
        tolerance.compare_e8(cb[rows], ref_bits, mag, 1024, f"grouped e8 expert {g}")
    assert (c[torch.from_numpy(layout < 0).to(gpu)].float().cpu() == 1536.0).all()
