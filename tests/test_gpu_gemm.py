"""GPU parity of bfp8_gemm against the oracle, for every schedule, on the page's test case,
the N = K = 4096 sweep, the hidden-5120 transformer linears and ragged tails."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from tests import tolerance
from tests.gpu_util import announce, bits, quant_gpu_checked

pytestmark = pytest.mark.gpu

SCHEDULES = ["auto", "small_m", "tiled"]


@pytest.fixture(autouse=True)
def _restore_schedule():
    yield
    bfp8.set_schedule("auto")


_weights = {}


def _weight_on(dev, key, make):
    if key not in _weights:
        w = make()
        _weights[key] = (w, w.q.to(dev), w.s.to(dev))
    return _weights[key]


def _run(sched, q_dev, s_dev, bq_dev, bs_dev, what, out=None):
    bfp8.set_schedule(sched)
    announce("gemm", what, "schedule", sched, "->", bfp8.schedule_for(q_dev.shape[0], bq_dev.shape[0], q_dev.shape[1]))
    c = bfp8.gemm(q_dev, s_dev, bq_dev, bs_dev, out=out)
    torch.cuda.synchronize()
    return c


def _sample_rows(m, count, seed):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, m - 1], rng.choice(m, count - 2, replace=False)]))


@pytest.mark.parametrize("sched", SCHEDULES)
def test_page2_case(gpu, sched):
    """M=83, N=576, K=7168: the vLLM test's shapes, seed and distributions (full output)."""
    a, w = workloads.page2_case()
    q, s, q_ref, s_ref = quant_gpu_checked(a, gpu, "page2")
    c = _run(sched, q, s, w.q.to(gpu), w.s.to(gpu), "page2 83x576x7168")
    rows, cols, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy())
    st = tolerance.compare(bits(c), ref_bits, mag, 7168, f"page2 {sched}")
    print(sched, st)


@pytest.mark.parametrize("m", workloads.SQUARE_SMALL_M)
@pytest.mark.parametrize("sched", SCHEDULES)
def test_square_small_m(gpu, m, sched):
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m}")
    c = _run(sched, q, s, bq, bs, f"square M={m}")
    rows, cols, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy())
    tolerance.compare(bits(c), ref_bits, mag, 4096, f"square M={m} {sched}")


@pytest.mark.parametrize("m", workloads.SQUARE_LARGE_M)
@pytest.mark.parametrize("sched", ["auto", "tiled"])
def test_square_large_m_sampled_rows(gpu, m, sched):
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m}")
    c = _run(sched, q, s, bq, bs, f"square M={m}")
    rows = _sample_rows(m, 40, seed=m)
    _, cols, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    tolerance.compare(bits(c)[rows], ref_bits, mag, 4096, f"square M={m} {sched}")


@pytest.mark.parametrize("m", [640, 768, 1536, 3072])
def test_square_between_sweep_sizes(gpu, m):
    """M between the sweep's powers of two, where the automatic plan runs one partial round of
    bigger tiles (128x128, 256x128 or 256x256) instead of two rounds of smaller ones."""
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m}")
    c = _run("auto", q, s, bq, bs, f"square M={m}")
    rows = _sample_rows(m, 40, seed=m + 1)
    _, cols, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    tolerance.compare(bits(c)[rows], ref_bits, mag, 4096, f"square M={m} auto")


@pytest.mark.parametrize("layer", list(workloads.TRANSFORMER_LAYERS))
@pytest.mark.parametrize("m", sorted(set(workloads.TRANSFORMER_M) | {32, 64, 256}))
def test_transformer_linears(gpu, layer, m):
    n, k = workloads.TRANSFORMER_LAYERS[layer]
    w, bq, bs = _weight_on(gpu, layer, lambda: workloads.transformer_weight(layer))
    q, s, q_ref, s_ref = quant_gpu_checked(workloads.transformer_act(layer, m), gpu, f"{layer} M={m}")
    c = _run("auto", q, s, bq, bs, f"{layer} M={m} N={n} K={k}")
    rows = _sample_rows(m, 24, seed=m + 7)
    rng = np.random.default_rng(n + m)
    cols = np.unique(np.concatenate([np.arange(128), np.arange(n - 130, n), rng.choice(n, 700, replace=False)]))
    _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows, cols=cols)
    tolerance.compare(bits(c)[np.ix_(rows, cols)], ref_bits, mag, k, f"{layer} M={m}")


def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A
    return torch.from_numpy(c)


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (7, 17, 256), (83, 136, 128), (129, 576, 384), (64, 200, 256),
                                   (65, 130, 512), (200, 40, 128), (83, 136, 1024), (129, 576, 2048)])
@pytest.mark.parametrize("sched", SCHEDULES)
def test_ragged_tails_with_padded_strides(gpu, m, n, k, sched):
    """Ragged M and N (partial 16-row, 128-row and weight-scale strips), padded row strides
    on every operand, and bytes outside the logical output left untouched."""
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = _random_codes(rng, (m, k + 32))
    b = _random_codes(rng, (n, k + 48))
    a_s = torch.from_numpy(rng.uniform(0.01, 2, (k // 128, m + 5)).astype(np.float32))
    b_s = torch.from_numpy(rng.uniform(1e-3, 1e-2, (-(-n // 128), k // 128 + 2)).astype(np.float32))
    ad, bd = a.to(gpu)[:, :k], b.to(gpu)[:, :k]
    asd = a_s.to(gpu)[:, :m].t()
    bsd = b_s.to(gpu)[:, :k // 128]
    c_full = torch.full((m, n + 9), -7.0, dtype=torch.bfloat16, device=gpu)
    c = _run(sched, ad, asd, bd, bsd, f"tails M={m} N={n} K={k}", out=c_full[:, :n])
    a_np, b_np = a[:, :k].numpy(), b[:, :k].numpy()
    as_np = a_s[:, :m].t().contiguous().numpy()
    bs_np = b_s[:, :k // 128].contiguous().numpy()
    rows, cols, ref_bits, mag = tolerance.reference(a_np, as_np, b_np, bs_np)
    mmax = tolerance.block_max_mass(a_np, as_np, b_np, bs_np, rows, cols)
    st = tolerance.compare(bits(c), ref_bits, mag, k, f"tails {m}x{n}x{k} {sched}", hw_block=mmax)
    print(st)
    assert (c_full[:, n:].float().cpu() == -7.0).all()


@pytest.mark.parametrize("m,n,k", [(640, 4000, 512), (769, 4112, 256), (1536, 4040, 512), (1583, 1320, 1024),
                                   (3000, 2056, 512), (2953, 5416, 1024)])
def test_tiled_launch_choices_ragged(gpu, m, n, k):
    """Shapes whose base plan leaves a partial last round, with ragged M and N and padded strides:
    the first five run fewer, bigger tiles (128x128 or 256x128) in one round, the last splits its
    columns (256x256 whole rounds, then the remaining 40 columns). Sampled rows, every column."""
    rng = np.random.default_rng(m + 3 * n + k)
    a = _random_codes(rng, (m, k + 32))
    b = _random_codes(rng, (n, k + 16))
    a_s = torch.from_numpy(rng.uniform(0.01, 2, (k // 128, m + 3)).astype(np.float32))
    b_s = torch.from_numpy(rng.uniform(1e-3, 1e-2, (-(-n // 128), k // 128 + 1)).astype(np.float32))
    ad, bd = a.to(gpu)[:, :k], b.to(gpu)[:, :k]
    asd = a_s.to(gpu)[:, :m].t()
    bsd = b_s.to(gpu)[:, :k // 128]
    c_full = torch.full((m, n + 8), -7.0, dtype=torch.bfloat16, device=gpu)
    c = _run("auto", ad, asd, bd, bsd, f"launch choice M={m} N={n} K={k}", out=c_full[:, :n])
    a_np, b_np = a[:, :k].numpy(), b[:, :k].numpy()
    as_np = a_s[:, :m].t().contiguous().numpy()
    bs_np = b_s[:, :k // 128].contiguous().numpy()
    rows = _sample_rows(m, 20, seed=m)
    _, cols, ref_bits, mag = tolerance.reference(a_np, as_np, b_np, bs_np, rows=rows)
    mmax = tolerance.block_max_mass(a_np, as_np, b_np, bs_np, rows, cols)
    tolerance.compare(bits(c)[rows], ref_bits, mag, k, f"launch choice {m}x{n}x{k}", hw_block=mmax)
    assert (c_full[:, n:].float().cpu() == -7.0).all()


def _code(v):
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


@pytest.mark.parametrize("sched", SCHEDULES)
def test_fp8_block_dot_alignment_window(gpu, sched):
    """The FP8 matrix-core block dot drops products far below the block's largest one.

    Row 0: 32 - 32 + 126 * 2**-9 (exact 0.24609375); row 1: the same small terms alone. With
    unit scales C is the raw block dot. Row 1 must be exact; row 0 may lose the small terms
    (the measured gfx950 behaviour) and must stay within the HW_BLOCK_ETA model."""
    k, n = 128, 16
    a = torch.zeros(2, k, dtype=torch.uint8)
    a[0, 0], a[0, 1] = _code(32.0), _code(-32.0)
    a[:, 2:] = _code(2.0**-9)
    b = torch.full((n, k), _code(1.0), dtype=torch.uint8)
    a_s = torch.ones(1, 2, dtype=torch.float32)
    b_s = torch.ones(1, 1, dtype=torch.float32)
    c = _run(sched, a.to(gpu), a_s.to(gpu).t(), b.to(gpu), b_s.to(gpu), "alignment window")
    got = c.float().cpu()
    exact = 126 * 2.0**-9
    assert (got[1] == exact).all()
    assert ((got[0] - exact).abs() <= tolerance.HW_BLOCK_ETA * 32.0).all()
    print(sched, "row0:", float(got[0, 0]), "exact:", exact)


@pytest.mark.parametrize("m,sched", [(9, "auto"), (256, "small_m"), (128, "auto"), (512, "tiled"), (2048, "auto")])
def test_run_to_run_bitwise_determinism(gpu, m, sched):
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    q, s, _, _ = quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m}")
    c1 = _run(sched, q, s, bq, bs, f"determinism M={m} run 1").clone()
    c2 = _run(sched, q, s, bq, bs, f"determinism M={m} run 2")
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_m_zero_and_rejections(gpu):
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    q = torch.zeros(0, 4096, dtype=torch.uint8, device=gpu)
    s = torch.zeros(32, 0, dtype=torch.float32, device=gpu).t()
    assert bfp8.gemm(q, s, bq, bs).shape == (0, 4096)
    q1 = torch.zeros(4, 4096 + 16, dtype=torch.uint8, device=gpu)[:, 1:4097]  # misaligned rows
    s1 = torch.ones(32, 4, dtype=torch.float32, device=gpu).t()
    with pytest.raises(ValueError):
        bfp8.gemm(q1, s1, bq, bs)
    q2 = torch.zeros(4, 200, dtype=torch.uint8, device=gpu)
    with pytest.raises(ValueError):
        bfp8.gemm(q2, s1, bq, bs)


def test_tile_plans_back_to_back_with_caller_workspace(gpu):
    """Tiled GEMMs whose plans differ (128x64, 128x128, 256x128 and 256x256 tiles, ragged M)
    run back to back with one caller-owned workspace; each must match the oracle."""
    w, bq, bs = _weight_on(gpu, "square", workloads.square_weight)
    sizes = [128, 160, 96, 600, 1024, 130, 2048, 4096, 128]
    need = max(bfp8._native.lib().bfp8_gemm_workspace_bytes(m, 4096, 4096) for m in sizes)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=gpu)
    bfp8.set_schedule("tiled")
    for m in sizes:
        q, s, q_ref, s_ref = quant_gpu_checked(workloads.square_act(m), gpu, f"square M={m}")
        announce("gemm", f"caller workspace M={m}")
        c = bfp8.gemm(q, s, bq, bs, workspace=ws)
        torch.cuda.synchronize()
        rows = _sample_rows(m, 16, seed=m + 1)
        _, _, ref_bits, mag = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
        tolerance.compare(bits(c)[rows], ref_bits, mag, 4096, f"caller workspace M={m}")
