"""GPU parity with a partial last K block (K % 128 != 0, K a multiple of 16).

The quantizer bit for bit (it writes no byte past K), and the dense GEMM on every schedule,
the grouped GEMM, the UE8M0 GEMM and the linear layer against the oracle. Operand rows are
padded to whole 128-byte blocks and the padding bytes hold NaN codes (0x7F, 0xFF): a kernel
that let one of them into a product would return NaN."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import linear, quant, ue8m0
from tests import tolerance
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu

NAN_CODES = (0x7F, 0xFF)


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


def _kp(k):
    return -(-k // 128) * 128


def _nan_padded(codes: torch.Tensor, dev, fill=0x7F) -> torch.Tensor:
    """[..., K] codes on dev in rows of Kp bytes whose bytes past K hold a NaN code."""
    *lead, k = codes.shape
    buf = torch.full((*lead, _kp(k)), fill, dtype=torch.uint8)
    buf[..., :k] = codes
    return buf.to(dev)[..., :k]


def _quant_nan_padded(x_cpu: torch.Tensor, dev, what: str):
    """quant_act into a q buffer prefilled with NaN codes; checks the codes and scales bit for bit
    and that the padding past K is untouched. Returns (q_dev, s_dev, q_ref, s_ref)."""
    m, k = x_cpu.shape
    announce("quant_act tail", what, m, k, x_cpu.dtype)
    q_buf = torch.full((m, _kp(k)), 0x7F, dtype=torch.uint8, device=dev)
    q, s = bfp8.quant_act(x_cpu.to(dev), q=q_buf[:, :k])
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x_cpu.float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().contiguous().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert (q_buf[:, k:].cpu() == 0x7F).all(), "the quantizer wrote past K"
    return q, s, q_ref, s_ref


@pytest.mark.parametrize("k", [16, 112, 144, 464, 1008])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_quant_partial_last_group(gpu, k, dtype):
    m = 37
    x = workloads.act_uniform(m, k, seed=k) if dtype == torch.float32 else workloads.act_normal_bf16(m, k, seed=k).to(dtype)
    _quant_nan_padded(x, gpu, f"{dtype}")


def test_quant_default_allocation_pads_rows(gpu):
    q, s = bfp8.quant_act(torch.zeros(3, 144, dtype=torch.bfloat16, device=gpu))
    assert q.shape == (3, 144) and q.stride(0) == 256 and s.shape == (3, 2)


def _rows(m, count, seed):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, m - 1], rng.choice(m, count - 2, replace=False)]))


@pytest.mark.parametrize("m,n,k", [(1, 200, 144), (37, 1000, 464), (300, 576, 1008), (2048, 4096, 4160),
                                   (4096, 4096, 1936), (5, 136, 16)])
@pytest.mark.parametrize("sched", ["auto", "small_m", "tiled"])
def test_gemm_partial_last_block(gpu, m, n, k, sched):
    """Ragged N, every tile plan of the tiled schedule (4096 x 4096 takes the 256 x 256 plan,
    run with 256 x 128 masked tiles), K tails of 16, 80, 112 and 64 bytes."""
    a = workloads.act_uniform(m, k, seed=m + k)
    q, s, q_ref, s_ref = _quant_nan_padded(a, gpu, f"gemm {m}x{n}x{k}")
    w = workloads.weight(n, k, seed=n + k)
    bq = _nan_padded(w.q, gpu, fill=NAN_CODES[(m + n) % 2])
    bfp8.set_schedule(sched)
    announce("gemm tail", m, n, k, sched, "->", bfp8.schedule_for(m, n, k))
    c = bfp8.gemm(q, s, bq, w.s.to(gpu))
    torch.cuda.synchronize()
    rows = _rows(m, 48, seed=k)
    r, cols, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    # K below one block: a few products per block, held to the matrix core's alignment window too
    hw = tolerance.block_max_mass(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows, cols) if k < 128 else None
    st = tolerance.compare(bits(c)[rows], ref_bits, mag, k, f"gemm tail {m}x{n}x{k} {sched}", hw_block=hw)
    print(sched, st)


@pytest.mark.parametrize("sched", ["small_m", "tiled"])
def test_gemm_f16_partial_last_block(gpu, sched):
    m, n, k = 64, 384, 464
    a = workloads.act_normal_bf16(m, k, seed=5)
    q, s, q_ref, s_ref = _quant_nan_padded(a, gpu, "gemm_f16")
    w = workloads.weight(n, k, seed=6)
    bfp8.set_schedule(sched)
    announce("gemm_f16 tail", m, n, k, sched)
    c = bfp8.gemm_f16(q, s, _nan_padded(w.q, gpu), w.s.to(gpu))
    torch.cuda.synchronize()
    from oracle import f16, gemm

    acc, _ = gemm.gemm_acc_ref(q_ref, s_ref, w.q.numpy(), w.s.numpy())
    mag = tolerance.masses(q_ref, s_ref, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
    got = c.cpu().view(torch.int16).numpy().view(np.uint16)
    tolerance.compare_f16(got, f16.to_bits(acc), mag, k, f"gemm_f16 tail {sched}")


def test_grouped_partial_last_block(gpu):
    g, n, k = 3, 384, 464
    layout = np.full(640, -1, np.int32)
    layout[0:100] = 0
    layout[128:384] = 2
    layout[384:500] = 1
    a = workloads.act_uniform(640, k, seed=7)
    q, s, q_ref, s_ref = _quant_nan_padded(a, gpu, "grouped")
    ws = [workloads.weight(n, k, seed=10 + i) for i in range(g)]
    bq = _nan_padded(torch.stack([w.q for w in ws]), gpu)
    bs = torch.stack([w.s for w in ws])
    announce("grouped tail", layout.size, n, k)
    c = bfp8.grouped_gemm_contiguous(q, s, bq, bs.to(gpu), torch.from_numpy(layout).to(gpu))
    torch.cuda.synchronize()
    got = bits(c)
    for e in range(g):
        rows = np.nonzero(layout == e)[0]
        w = ws[e]
        _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
        tolerance.compare(got[rows], ref_bits, mag, k, f"grouped tail expert {e}")


@pytest.mark.parametrize("sched", ["small_m", "tiled"])
def test_ue8m0_partial_last_block(gpu, sched):
    m, n, k = 96, 520, 1008
    a = workloads.act_uniform(m, k, seed=8)
    announce("quant_act_ue8m0 tail", m, k)
    q_buf = torch.full((m, _kp(k)), 0xFF, dtype=torch.uint8, device=gpu)
    q, e = bfp8.quant_act_ue8m0(a.to(gpu), q=q_buf[:, :k])
    torch.cuda.synchronize()
    q_ref, e_ref = ue8m0.quant_act_ue8m0_ref(a.numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(e.cpu().contiguous().numpy(), e_ref)
    assert (q_buf[:, k:].cpu() == 0xFF).all()
    w = workloads.weight_ue8m0(n, k, seed=9)
    bfp8.set_schedule(sched)
    announce("gemm_ue8m0 tail", m, n, k, sched)
    c = bfp8.gemm_ue8m0(q, e, _nan_padded(w.q, gpu), bfp8.ue8m0_scales(w.s.to(gpu)))
    torch.cuda.synchronize()
    _, _, ref_bits, mag = tolerance.reference_e8(q_ref, e_ref, w.q.numpy(), w.s.numpy())
    tolerance.compare_e8(bits(c), ref_bits, mag, k, f"gemm_ue8m0 tail {sched}")


@pytest.mark.parametrize("m", [3, 300])
def test_linear_partial_last_block(gpu, m):
    n, k = 640, 464
    x = workloads.act_normal_bf16(m, k, seed=m)
    w = workloads.weight(n, k, seed=11)
    rng = np.random.default_rng(12)
    bias = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    announce("linear tail", m, n, k)
    y = bfp8.linear(x.to(gpu), _nan_padded(w.q, gpu), w.s.to(gpu), bias.to(gpu))
    torch.cuda.synchronize()
    out_ref, c_ref, q, s = linear.linear_ref(x.float().numpy(), w.q.numpy(), w.s.numpy(), bias=bias.float().numpy())
    mag = tolerance.masses(q, s, w.q.numpy(), w.s.numpy(), np.arange(m), np.arange(n))
    tolerance.compare_linear(bits(y), out_ref, c_ref, mag, k, f"linear tail m={m}")


def test_pad_k_layout(gpu):
    codes = torch.randint(0, 256, (2, 5, 144), dtype=torch.uint8)
    p = bfp8.pad_k(codes.to(gpu))
    assert p.shape == codes.shape and p.stride() == (5 * 256, 256, 1)
    assert torch.equal(p.cpu(), codes)
    assert bfp8.pad_k(p) is p  # already laid out so: no copy


def test_nn_weights_partial_last_block(gpu):
    """NN expert weights [G, K, N] with K % 128 != 0: converted into rows of whole blocks, then
    the grouped GEMM against the oracle written on the NN operand."""
    g, n, k = 2, 264, 464
    ws = [workloads.weight(n, k, seed=40 + i) for i in range(g)]
    w_nn = torch.stack([w.q.t().contiguous() for w in ws])
    s_nn = torch.stack([w.s.t().contiguous() for w in ws])
    announce("nn_to_nt_weights tail", tuple(w_nn.shape))
    w_nt, s_nt = bfp8.nn_to_nt_weights(w_nn.to(gpu), s_nn.to(gpu))
    torch.cuda.synchronize()
    assert w_nt.stride(1) == _kp(k)
    np.testing.assert_array_equal(w_nt.cpu().numpy(), w_nn.numpy().transpose(0, 2, 1))
    layout = np.full(384, -1, np.int32)
    layout[:77] = 1
    layout[128:300] = 0
    x = workloads.act_normal_bf16(384, k, seed=41)
    q, s, q_ref, s_ref = _quant_nan_padded(x, gpu, "nn tail activations")
    announce("grouped nn tail", n, k)
    c = bfp8.grouped_gemm_contiguous(q, s, w_nt, s_nt, torch.from_numpy(layout).to(gpu))
    torch.cuda.synchronize()
    from oracle import bf16, gemm

    rows, acc = gemm.grouped_gemm_contiguous_nn_acc_ref(q_ref, s_ref, w_nn.numpy(), s_nn.numpy(), layout)
    got = bits(c)[rows]
    mag = tolerance.Mass.zeros(acc.shape)
    for e in range(g):
        sel = layout[rows] == e
        mag[sel] = tolerance.masses(q_ref, s_ref, ws[e].q.numpy(), ws[e].s.numpy(), rows[sel], np.arange(n))
    tolerance.compare(got, bf16.to_bits(acc), mag, k, "grouped nn tail")
