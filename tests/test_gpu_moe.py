"""GPU parity of the MoE chain against the oracle: the dispatch layout, the gathered quantizer,
SwiGLU + quantization and the combine bit for bit on seeded inputs; the fused forward equal to its
steps called one by one, and against the oracle's forward within a derived bound."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from oracle import bf16, e4m3, moe, quant
from tests.gpu_util import announce, bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("t,k,e,sent", [(512, 8, 16, 0.0), (700, 6, 64, 0.05), (3, 1, 1, 0.0), (2000, 1, 1024, 0.0),
                                        (1, 4, 5, 0.5)])
def test_dispatch_layout(gpu, t, k, e, sent):
    ids, _ = workloads.moe_routing(t, k, e, seed=t + e, sentinel_frac=sent)
    announce("moe_dispatch", t, k, e, sent)
    row_of_pair, pair_of_row, layout, start = bfp8.moe_dispatch(ids.to(gpu), e)
    torch.cuda.synchronize()
    r_ref, p_ref, l_ref, s_ref = moe.layout_ref(ids.numpy(), e, 128)
    n = l_ref.size
    assert layout.numel() >= n and layout.numel() % 128 == 0
    np.testing.assert_array_equal(row_of_pair.cpu().numpy(), r_ref)
    np.testing.assert_array_equal(start.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(layout.cpu().numpy()[:n], l_ref)
    np.testing.assert_array_equal(pair_of_row.cpu().numpy()[:n], p_ref)
    assert (layout.cpu().numpy()[n:] == -1).all() and (pair_of_row.cpu().numpy()[n:] == -1).all()


def test_dispatch_is_deterministic(gpu):
    ids, _ = workloads.moe_routing(4096, 8, 32, seed=1)
    ids_d = ids.to(gpu)
    a = bfp8.moe_dispatch(ids_d, 32)
    b = bfp8.moe_dispatch(ids_d, 32)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_act_gather(gpu, dtype):
    t, k, h = 37, 3, 384
    x = workloads.act_normal_bf16(t, h, seed=11).to(dtype) if dtype == torch.bfloat16 else workloads.act_uniform(t, h, 12)
    rows = 256
    rng = np.random.default_rng(13)
    src = np.full(rows, -1, dtype=np.int32)
    used = rng.choice(rows, 90, replace=False)
    src[used] = rng.integers(0, t * k, 90)
    announce("quant_act_gather", dtype, rows)
    q, s = bfp8.quant_act_gather(x.to(gpu), torch.from_numpy(src).to(gpu), k)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x.float().numpy()[src[used] // k])
    np.testing.assert_array_equal(q.cpu().numpy()[used], q_ref)
    np.testing.assert_array_equal(s.cpu().numpy()[used].view(np.uint32), s_ref.view(np.uint32))


def test_swiglu_quant(gpu):
    m, i = 300, 512
    rng = np.random.default_rng(14)
    proj = torch.from_numpy(rng.standard_normal((m, 2 * i)).astype(np.float32) * 4).to(torch.bfloat16)
    proj[7] *= 2.0**-80  # tiny values: subnormal products inside the gate
    proj[8, :i] = -200.0  # silu underflows to -0
    layout = np.where(rng.random(m) < 0.2, -1, 0).astype(np.int32)
    announce("swiglu_quant", m, i)
    q, s = bfp8.swiglu_quant(proj.to(gpu), torch.from_numpy(layout).to(gpu))
    torch.cuda.synchronize()
    h = moe.swiglu_ref(proj.view(torch.int16).numpy().view(np.uint16))
    q_ref, s_ref = quant.quant_act_ref(bf16.from_bits(h).astype(np.float32))
    ok = layout >= 0
    np.testing.assert_array_equal(q.cpu().numpy()[ok], q_ref[ok])
    np.testing.assert_array_equal(s.cpu().numpy()[ok].view(np.uint32), s_ref[ok].view(np.uint32))


def test_combine(gpu):
    t, k, h = 129, 4, 1024
    rng = np.random.default_rng(15)
    rows = 700
    out = torch.from_numpy(rng.standard_normal((rows, h)).astype(np.float32) * 3).to(torch.bfloat16)
    row_of_pair = rng.choice(rows - 10, t * k, replace=False).astype(np.int32)
    row_of_pair[rng.random(t * k) < 0.1] = -1
    out[rows - 10:] = float("nan")  # rows nobody references
    _, w = workloads.moe_routing(t, k, 8, seed=16)
    announce("moe_combine", t, k, h)
    y = bfp8.moe_combine(out.to(gpu), torch.from_numpy(row_of_pair).to(gpu), w.to(gpu))
    torch.cuda.synchronize()
    want = moe.combine_ref(out.view(torch.int16).numpy().view(np.uint16), row_of_pair, w.numpy(), t, k)
    np.testing.assert_array_equal(bits(y), want)


_chain = {}


def _chain_inputs(dev, t=192, k=4, e=8, h=256, i=256, sent=0.05):
    key = (t, k, e, h, i, sent)
    if key not in _chain:
        x = workloads.act_normal_bf16(t, h, seed=21)
        ids, w = workloads.moe_routing(t, k, e, seed=22, sentinel_frac=sent)
        wts = workloads.moe_experts(e, h, i, seed=23)
        _chain[key] = (x, ids, w, wts, [a.to(dev) for a in (x, ids, w, *wts)])
    return _chain[key]


def test_forward_equals_its_steps(gpu):
    """bfp8_moe_forward, bit for bit, equals dispatch -> gathered quantization -> grouped GEMM ->
    SwiGLU + quantization -> grouped GEMM -> combine called one by one."""
    x, ids, w, wts, (xd, idsd, wd, wu, su, wdn, sdn) = _chain_inputs(gpu)
    e = wu.shape[0]
    announce("moe_forward fused vs steps")
    y = bfp8.moe_forward(xd, idsd, wd, wu, su, wdn, sdn)
    row_of_pair, pair_of_row, layout, _ = bfp8.moe_dispatch(idsd, e)
    q, s = bfp8.quant_act_gather(xd, pair_of_row, ids.shape[1])
    proj = bfp8.grouped_gemm_contiguous(q, s, wu, su, layout)
    q2, s2 = bfp8.swiglu_quant(proj, layout)
    out = bfp8.grouped_gemm_contiguous(q2, s2, wdn, sdn, layout)
    y2 = bfp8.moe_combine(out, row_of_pair, wd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def _down_mass(x, ids, w, wts):
    """Per output element, sum_j |bf16(w_j)| * sum_i |h_i| |W_down[i]| |Bs| of the oracle (float64)."""
    w_up, s_up, w_down, s_down = (a.numpy() for a in wts)
    t, k = ids.shape
    mass = np.zeros((t, w_down.shape[1]))
    for p in range(t * k):
        g = int(ids.numpy().reshape(-1)[p])
        if g < 0 or g >= w_up.shape[0]:
            continue
        _, _, h = moe.expert_mlp_ref(x.float().numpy()[p // k][None], w_up[g], s_up[g], w_down[g], s_down[g])
        hv = np.abs(bf16.from_bits(h)[0])
        wv = np.abs(e4m3.decode(w_down[g]))  # [H, I]
        sc = np.repeat(np.repeat(np.abs(s_down[g]), 128, axis=0), 128, axis=1)[: wv.shape[0], : wv.shape[1]]
        mass[p // k] += abs(float(w.numpy().reshape(-1)[p])) * (wv * sc) @ hv
    return mass


def test_forward_against_oracle(gpu):
    """The fused forward against the oracle's forward on the same inputs. The two sides agree up to
    the GEMMs' rounding; where that flips a code of the second quantization, the element moves by
    at most one e4m3 step (2^-3 of |h|) of that term, so the bound is 2^-2 of the down product's
    absolute mass plus 2 bf16 ulp; the mean relative error must stay below 1e-2."""
    x, ids, w, wts, (xd, idsd, wd, wu, su, wdn, sdn) = _chain_inputs(gpu)
    announce("moe_forward vs oracle")
    y = bfp8.moe_forward(xd, idsd, wd, wu, su, wdn, sdn)
    torch.cuda.synchronize()
    ref = moe.moe_forward_ref(x.float().numpy(), ids.numpy(), w.numpy(), *(a.numpy() for a in wts))
    got_v, ref_v = bf16.from_bits(bits(y)), bf16.from_bits(ref)
    d = np.abs(got_v - ref_v)
    assert np.isfinite(got_v).all()
    rel_mean = d.mean() / np.abs(ref_v).mean()
    mass = _down_mass(x, ids, w, wts)
    bound = 2.0**-2 * mass + 2 * bf16.ulp(ref_v)
    print({"rel_mean": float(rel_mean), "exact_frac": float(np.mean(bits(y) == ref)), "max_over_mass": float((d / (mass + 1e-30)).max())})
    assert rel_mean < 1e-2
    assert (d <= bound).all()


def test_forward_all_sentinels_and_single_token(gpu):
    x, ids, w, wts, (xd, idsd, wd, wu, su, wdn, sdn) = _chain_inputs(gpu)
    e = wu.shape[0]
    announce("moe_forward sentinels")
    y = bfp8.moe_forward(xd[:5], torch.full((5, 4), e, dtype=torch.int32, device=gpu), wd[:5], wu, su, wdn, sdn)
    torch.cuda.synchronize()
    assert (y.float() == 0).all()
    y1 = bfp8.moe_forward(xd[:1], idsd[:1], wd[:1], wu, su, wdn, sdn)
    torch.cuda.synchronize()
    ref = moe.moe_forward_ref(x.float().numpy()[:1], ids.numpy()[:1], w.numpy()[:1], *(a.numpy() for a in wts))
    assert np.abs(bf16.from_bits(bits(y1)) - bf16.from_bits(ref)).mean() <= 1e-2 * np.abs(bf16.from_bits(ref)).mean() + 1e-30
