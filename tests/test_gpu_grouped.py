"""GPU parity of bfp8_grouped_gemm_contiguous against the oracle (M-grouped contiguous MoE GEMM)."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from tests import tolerance
from tests.gpu_util import announce, bits, quant_gpu_checked

pytestmark = pytest.mark.gpu

_moe = {}


def _moe_on(dev):
    if "case" not in _moe:
        case = workloads.moe_case()
        bq = torch.stack([w.q for w in case.weights])
        bs = torch.stack([w.s for w in case.weights])
        _moe["case"] = (case, bq, bs, bq.to(dev), bs.to(dev))
    return _moe["case"]


def _grouped(q, s, bq, bs, layout, what, out=None):
    announce("grouped_gemm", what, tuple(q.shape), tuple(bq.shape))
    c = bfp8.grouped_gemm_contiguous(q, s, bq, bs, layout, out=out)
    torch.cuda.synchronize()
    return c


def _check_rows(c_bits, q_ref, s_ref, bq, bs, layout, rows_per_group, cols, what):
    rng = np.random.default_rng(17)
    k = q_ref.shape[1]
    for g in np.unique(layout[layout >= 0]):
        rows = np.nonzero(layout == g)[0]
        rows = np.unique(np.concatenate([rows[:1], rows[-1:], rng.choice(rows, min(rows_per_group, rows.size),
                                                                          replace=False)]))
        _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, bq[g], bs[g], rows=rows, cols=cols)
        tolerance.compare(c_bits[np.ix_(rows, cols)], ref_bits, mag, k, f"{what} expert {g}")


def test_moe_config(gpu):
    """16 experts, N=4096, K=7168, 4096 tokens with Dirichlet(1) counts, 128-row padding."""
    case, bq, bs, bq_d, bs_d = _moe_on(gpu)
    q, s, q_ref, s_ref = quant_gpu_checked(case.act, gpu, "moe activations")
    layout = case.layout.numpy()
    lay_d = case.layout.to(gpu)
    sentinel = torch.full((layout.size, 4096), 1536.0, dtype=torch.bfloat16, device=gpu)
    c = _grouped(q, s, bq_d, bs_d, lay_d, "moe config", out=sentinel)
    cb = bits(c)
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(4032, 4096), rng.choice(4096, 400, replace=False)]))
    _check_rows(cb, q_ref, s_ref, bq.numpy(), bs.numpy(), layout, 6, cols, "moe")
    # padding rows are not written
    pad = layout < 0
    assert (c[torch.from_numpy(pad).to(gpu)].float().cpu() == 1536.0).all()


def test_down_projection_shape(gpu):
    """The MoE chain's down projection: 16 experts with weights [N = 7168, K = 2048], the grouped
    configuration's Dirichlet(1) counts over 4096 tokens, 128-row padding."""
    case = workloads.moe_case(n=7168, k=2048, seed=6)
    bq = torch.stack([w.q for w in case.weights])
    bs = torch.stack([w.s for w in case.weights])
    q, s, q_ref, s_ref = quant_gpu_checked(case.act, gpu, "moe down activations")
    layout = case.layout.numpy()
    out = torch.full((layout.size, 7168), 1536.0, dtype=torch.bfloat16, device=gpu)
    c = _grouped(q, s, bq.to(gpu), bs.to(gpu), case.layout.to(gpu), "moe down", out=out)
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(7104, 7168), rng.choice(7168, 400, replace=False)]))
    _check_rows(bits(c), q_ref, s_ref, bq.numpy(), bs.numpy(), layout, 6, cols, "moe down")
    assert (c[torch.from_numpy(layout < 0).to(gpu)].float().cpu() == 1536.0).all()


def test_poisoned_padding_rows_and_empty_blocks(gpu):
    """Padding rows full of NaN codes and NaN scales, plus a trailing all-padding block: valid rows
    are bitwise unchanged and no padding row is written."""
    g_count, n, k = 3, 384, 512
    counts = np.array([130, 0, 45])
    layout = workloads.moe_layout(counts)
    layout = np.concatenate([layout, np.full(128, -1, np.int32)])  # a block of padding only
    m = layout.size
    ws = [workloads.weight(n, k, seed=900 + g) for g in range(g_count)]
    bq = torch.stack([w.q for w in ws])
    bs = torch.stack([w.s for w in ws])
    x = workloads.act_normal_bf16(m, k, seed=77)
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, "grouped small")
    bq_d, bs_d, lay_d = bq.to(gpu), bs.to(gpu), torch.from_numpy(layout).to(gpu)
    c_clean = _grouped(q, s, bq_d, bs_d, lay_d, "clean").clone()
    pad = torch.from_numpy(layout < 0).to(gpu)
    q_p = q.clone()
    q_p[pad] = 0x7F
    s_p = s.clone()
    s_p[pad] = float("nan")
    out = torch.full((m, n), -3.0, dtype=torch.bfloat16, device=gpu)
    c_p = _grouped(q_p, s_p, bq_d, bs_d, lay_d, "poisoned", out=out)
    valid = ~pad
    assert torch.equal(c_p[valid].view(torch.int16), c_clean[valid].view(torch.int16))
    assert (c_p[pad].float() == -3.0).all()
    _check_rows(bits(c_clean), q_ref, s_ref, bq.numpy(), bs.numpy(), layout, 200, np.arange(n), "grouped small")


def test_mixed_expert_blocks_equal_dense(gpu):
    """Experts of 256, 128, 384, 0 and 200 rows, then a block of padding only: 128-row blocks e0 e0
    e1 e2 e2 e2 e4 e4 (the last 72 rows + padding) and one skipped block, so that the expert changes
    inside a 256-row tile, one expert is empty and the last tiles are part or all padding. Every
    valid row against the oracle, padding rows unwritten, and each expert's rows bit-equal to a
    dense GEMM of those rows with its weights."""
    g_count, n, k = 5, 512, 1024
    counts = np.array([256, 128, 384, 0, 200])
    layout = np.concatenate([workloads.moe_layout(counts), np.full(128, -1, np.int32)])
    m = layout.size
    assert m == 9 * 128
    ws = [workloads.weight(n, k, seed=950 + g) for g in range(g_count)]
    bq = torch.stack([w.q for w in ws])
    bs = torch.stack([w.s for w in ws])
    x = workloads.act_normal_bf16(m, k, seed=951)
    x[torch.from_numpy(layout < 0)] = 0
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, "mixed blocks")
    out = torch.full((m, n), -7.0, dtype=torch.bfloat16, device=gpu)
    c = _grouped(q, s, bq.to(gpu), bs.to(gpu), torch.from_numpy(layout).to(gpu), "mixed blocks", out=out)
    cb = bits(c)
    assert (c[torch.from_numpy(layout < 0).to(gpu)].float() == -7.0).all()
    _check_rows(cb, q_ref, s_ref, bq.numpy(), bs.numpy(), layout, 400, np.arange(n), "mixed blocks")
    # the tiled dense kernel adds every output's K blocks in the same order as the grouped one
    bfp8.set_schedule("tiled")
    try:
        for g in np.unique(layout[layout >= 0]):
            rows = torch.from_numpy(np.nonzero(layout == g)[0]).to(gpu)
            s_g = s[rows].t().contiguous().t()  # group-major, as quant_act lays scales out
            d = bfp8.gemm(q[rows].contiguous(), s_g, ws[g].q.to(gpu), ws[g].s.to(gpu))
            torch.cuda.synchronize()
            assert torch.equal(d.view(torch.int16), c[rows].view(torch.int16)), f"expert {g}"
    finally:
        bfp8.set_schedule("auto")


def test_single_group_equals_dense_tiled(gpu):
    """G = 1 with no padding is the dense product. At 2048 x 2048 the dense tiled plan fills the
    chip without splitting K, so both sum every output block by block in the same order and
    must agree bitwise (a split-K plan adds its partial sums in another order)."""
    m, n, k = 2048, 2048, 1024
    assert bfp8.schedule_for(m, n, k) == "tiled" and bfp8._native.lib().bfp8_gemm_workspace_bytes(m, n, k) == 0
    w = workloads.weight(n, k, seed=31)
    x = workloads.act_normal_bf16(m, k, seed=32)
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, "single group")
    bq_d, bs_d = w.q.to(gpu), w.s.to(gpu)
    lay = torch.zeros(m, dtype=torch.int32, device=gpu)
    c_g = _grouped(q, s, bq_d[None], bs_d[None], lay, "G=1")
    bfp8.set_schedule("tiled")
    try:
        c_d = bfp8.gemm(q, s, bq_d, bs_d)
        torch.cuda.synchronize()
    finally:
        bfp8.set_schedule("auto")
    assert torch.equal(c_g.view(torch.int16), c_d.view(torch.int16))
    _check_rows(bits(c_g), q_ref, s_ref, w.q.numpy()[None], w.s.numpy()[None], np.zeros(m, np.int32), 24,
                np.arange(n), "single group")


def test_grouped_rejections(gpu):
    q = torch.zeros(100, 256, dtype=torch.uint8, device=gpu)
    s = torch.ones(2, 100, dtype=torch.float32, device=gpu).t()
    bq = torch.zeros(2, 128, 256, dtype=torch.uint8, device=gpu)
    bs = torch.ones(2, 1, 2, dtype=torch.float32, device=gpu)
    lay = torch.zeros(100, dtype=torch.int32, device=gpu)
    with pytest.raises(ValueError):  # M % 128 != 0
        bfp8.grouped_gemm_contiguous(q, s, bq, bs, lay)



def test_nn_weights_converted_once(gpu):
    """NN expert weights [G, K, N] (the page's transposed experts): the conversion to [G, N, K] is
    bit-exact, and the grouped GEMM on the converted weights matches the NN oracle."""
    from oracle import gemm

    g_count, n, k = 3, 200, 384
    rng = np.random.default_rng(90)
    ws = [workloads.weight(n, k, seed=91 + g) for g in range(g_count)]
    w_nn = torch.stack([w.q.t().contiguous() for w in ws])  # [G, K, N]
    s_nn = torch.stack([w.s.t().contiguous() for w in ws])  # [G, K/128, ceil(N/128)]
    announce("nn_to_nt_weights", tuple(w_nn.shape))
    w_nt, s_nt = bfp8.nn_to_nt_weights(w_nn.to(gpu), s_nn.to(gpu))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w_nt.cpu().numpy(), w_nn.numpy().transpose(0, 2, 1))
    np.testing.assert_array_equal(s_nt.cpu().numpy(), s_nn.numpy().transpose(0, 2, 1))
    layout = np.concatenate([np.full(128, 2, np.int32), np.full(90, 0, np.int32), np.full(38, -1, np.int32),
                             np.full(128, 1, np.int32)])
    x = workloads.act_normal_bf16(layout.size, k, seed=95)
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, "nn activations")
    c = _grouped(q, s, w_nt, s_nt, torch.from_numpy(layout).to(gpu), "nn weights")
    rows, acc = gemm.grouped_gemm_contiguous_nn_acc_ref(q_ref, s_ref, w_nn.numpy(), s_nn.numpy(), layout)
    from oracle import bf16
    mag = tolerance.Mass.zeros(acc.shape)
    for g in range(g_count):
        sel = np.nonzero(layout[rows] == g)[0]
        mag[sel] = tolerance.masses(q_ref, s_ref, ws[g].q.numpy(), ws[g].s.numpy(), rows[sel], np.arange(n))
    tolerance.compare(bits(c)[rows], bf16.to_bits(acc), mag, k, "grouped nn")
