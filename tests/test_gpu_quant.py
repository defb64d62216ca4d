"""GPU parity of bfp8_quant_act against the oracle: bit-exact codes and scales."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import e4m3, quant
from tests.gpu_util import announce, quant_gpu_checked
from tests.test_oracle_quant import near_tie_rows

pytestmark = pytest.mark.gpu


def test_page2_activations(gpu):
    a, _ = workloads.page2_case()
    quant_gpu_checked(a, gpu, "page2 M=83 K=7168 fp32")


@pytest.mark.parametrize("m", [1, 9, 256, 2048])
def test_square_sweep_activations(gpu, m):
    quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m} K=4096 fp32")


@pytest.mark.parametrize("layer,m", [("qkv", 16), ("down", 128), ("o_proj", 2048)])
def test_transformer_activations_bf16(gpu, layer, m):
    quant_gpu_checked(workloads.transformer_act(layer, m), gpu, f"{layer} M={m} bf16")


def test_moe_activations_bf16(gpu):
    case = workloads.moe_case(with_weights=False)
    quant_gpu_checked(case.act, gpu, f"moe M_pad={case.act.shape[0]} K=7168 bf16")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_wide_mapping_partial_group_and_strided_rows(gpu, dtype):
    """32768 groups and more take 8 lanes per group (16 elements per lane): here with a partial
    last group (K = 16400 = 128 * 128 + 16) and rows 48 elements wider than K."""
    m, k = 300, 16400
    assert m * -(-k // 128) >= 32768
    rng = np.random.default_rng(31)
    full = torch.from_numpy((rng.standard_normal((m, k + 48)) * 3).astype(np.float32)).to(dtype)
    announce("quant_act wide", dtype, m, k, "strided")
    x_dev = full.to(gpu)[:, :k]
    assert x_dev.stride(0) == k + 48
    q, s = bfp8.quant_act(x_dev)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(full[:, :k].float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy()[:, :k], q_ref)
    np.testing.assert_array_equal(s.cpu().contiguous().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_wide_mapping_gather(gpu):
    """The gathered quantizer (MoE dispatch rows) on 4800 rows x 8 groups, with skipped rows."""
    t, top_k, h = 600, 8, 1024
    x = workloads.act_normal_bf16(t, h, seed=41)
    rows = t * top_k
    rng = np.random.default_rng(42)
    src = rng.permutation(rows).astype(np.int32)
    src[rng.choice(rows, 300, replace=False)] = -1
    used = src >= 0
    announce("quant_act_gather wide", rows, h)
    q, s = bfp8.quant_act_gather(x.to(gpu), torch.from_numpy(src).to(gpu), top_k)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x.float().numpy()[src[used] // top_k])
    np.testing.assert_array_equal(q.cpu().numpy()[used], q_ref)
    np.testing.assert_array_equal(s.cpu().numpy()[used].view(np.uint32), s_ref.view(np.uint32))


def test_near_e4m3_ties(gpu):
    """Quotients within a few float32 ulps of e4m3 rounding midpoints: a reciprocal-multiply
    or a wrongly rounded divide changes codes here."""
    x = torch.from_numpy(near_tie_rows(n_rows=64, seed=21))
    quant_gpu_checked(x, gpu, "near-tie rows")


def test_every_rounding_boundary_and_strided_float32(gpu):
    """With amax = 448 the scale is exactly 1, so the codes are the e4m3 encoding of x itself:
    every e4m3 value, midpoint and neighbouring float32, then every 97th float32 <= 448."""
    pos = np.sort(e4m3.decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids]).astype(np.float32)
    vals = [base]
    up, dn = base, base
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up, dn]
    v = np.concatenate(vals)
    v = v[(v >= 0) & (v <= 448)]
    limit = int(np.array([448.0], np.float32).view(np.uint32)[0])
    strided = np.arange(0, limit + 1, 97, dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, -v, strided, -strided]).astype(np.float32)
    per_row = 127
    rows = -(-v.size // per_row)
    v = np.concatenate([v, np.zeros(rows * per_row - v.size, np.float32)]).reshape(rows, per_row)
    x = np.concatenate([np.full((rows, 1), 448.0, np.float32), v], axis=1)
    quant_gpu_checked(torch.from_numpy(x), gpu, f"boundary sweep rows={rows}")


def test_zero_groups_signed_zeros_and_strides(gpu):
    """All-zero groups (scale floor), negative zeros, padded row strides for x, q and the scales."""
    m, k = 5, 384
    x_full = torch.zeros(m, k + 64, dtype=torch.float32)
    x_full[1, :128] = torch.linspace(-3, 3, 128)
    x_full[2, 5] = -0.0
    x_full[3, 300] = 1e-30
    x_full[4, :k] = workloads.act_uniform(1, k, seed=3)[0]
    x = x_full[:, :k]  # row stride 448 elements
    announce("quant_act strides", m, k)
    xd = x_full.to(gpu)[:, :k]
    q_buf = torch.full((m, k + 32), 0xAB, dtype=torch.uint8, device=gpu)
    s_buf = torch.full((k // 128, m + 3), -1.0, dtype=torch.float32, device=gpu)
    q, s = bfp8.quant_act(xd, q=q_buf[:, :k], scales=s_buf[:, :m].t())
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x.numpy())
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().contiguous().numpy().view(np.uint32), s_ref.view(np.uint32))
    # bytes past the logical extents are untouched
    assert (q_buf[:, k:].cpu() == 0xAB).all()
    assert (s_buf[:, m:].cpu() == -1.0).all()


def test_m_zero_is_a_noop(gpu):
    x = torch.zeros(0, 256, dtype=torch.float32, device=gpu)
    q, s = bfp8.quant_act(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_rejects_bad_arguments(gpu):
    x = torch.zeros(4, 200, dtype=torch.float32, device=gpu)
    with pytest.raises(NotImplementedError):
        bfp8.quant_act(x)  # K % 128 != 0
    x64 = torch.zeros(4, 256, dtype=torch.float64, device=gpu)
    with pytest.raises(NotImplementedError):
        bfp8.quant_act(x64)
    xo = torch.zeros(4, 257, dtype=torch.float32, device=gpu)[:, 1:]  # misaligned base
    with pytest.raises(ValueError):
        bfp8.quant_act(xo)
