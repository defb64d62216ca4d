"""GPU parity of the persistent schedule (by override only: the tiled kernel measured faster):
the oracle on sampled rows, and bit-equality with the tiled schedule, which sums every output's
K blocks in the same order (only the seam between a workgroup's tiles differs). Shapes with one
and two tiles per workgroup, ragged M and N (including an N that ends inside an 8-column
store), one to three K blocks, a column-split plan, a bias, and run-to-run determinism."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from tests import tolerance
from tests.gpu_util import announce, bits, quant_gpu_checked

pytestmark = pytest.mark.gpu


def _run(sched, q, s, wq, ws, out=None):
    bfp8.set_schedule(sched)
    try:
        c = bfp8.gemm(q, s, wq, ws, out=out)
        torch.cuda.synchronize()
    finally:
        bfp8.set_schedule("auto")
    return c


def test_persistent_only_by_override():
    for m in (8192, 7680, 16384):
        assert bfp8.schedule_for(m, 4096, 4096) == "tiled"
    bfp8.set_schedule("persistent")
    try:
        assert bfp8.schedule_for(8192, 4096, 4096) == "persistent"
    finally:
        bfp8.set_schedule("auto")


# Every shape's plan runs 256 x 256 tiles (a column split's lead launch where the tiles do not
# fill whole rounds): two tiles per workgroup with ragged M; two to three with ragged M; N ending
# inside an 8-column store with two K blocks; one K block; three K blocks.
@pytest.mark.parametrize("m,n,k", [(8192, 4096, 4096), (8192 + 77, 3968, 1024), (12288 + 100, 4096, 256),
                                   (2048, 10240, 5120),
                                   (8192, 3999, 256), (8448, 2048, 128), (16384, 1280, 384)])
def test_persistent_equals_tiled_and_oracle(gpu, m, n, k):
    w = workloads.weight(n, k, seed=60 + m % 97)
    x = workloads.act_uniform(m, k, seed=61 + n % 89)
    q, s, q_ref, s_ref = quant_gpu_checked(x, gpu, f"persistent {m}x{n}x{k}")
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    announce("gemm persistent vs tiled", m, n, k)
    if n % 8:
        # ldc a multiple of 8 (16-byte rows), N ending inside an 8-column store
        buf_p = torch.full((m, n + 8 - n % 8), -5.0, dtype=torch.bfloat16, device=gpu)
        buf_t = buf_p.clone()
        c_p = _run("persistent", q, s, wq, ws, out=buf_p[:, :n])
        c_t = _run("tiled", q, s, wq, ws, out=buf_t[:, :n])
        assert (buf_p[:, n:].float() == -5.0).all(), "bytes past N written"
    else:
        c_p = _run("persistent", q, s, wq, ws)
        c_t = _run("tiled", q, s, wq, ws)
    assert torch.equal(c_p.view(torch.int16), c_t.view(torch.int16))
    rng = np.random.default_rng(m + n)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 40, replace=False)]))
    _, _, ref_bits, mass = tolerance.reference(q_ref, s_ref, w.q.numpy(), w.s.numpy(), rows=rows)
    tolerance.compare(bits(c_p)[rows], ref_bits, mass, k, f"persistent {m}x{n}x{k}")


def test_persistent_is_deterministic(gpu):
    m, n, k = 8192, 4096, 2048
    w = workloads.weight(n, k, seed=70)
    x = workloads.act_uniform(m, k, seed=71)
    q, s = bfp8.quant_act(x.to(gpu))
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    announce("gemm persistent determinism", m, n, k)
    a = _run("persistent", q, s, wq, ws)
    b = _run("persistent", q, s, wq, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_persistent_linear_with_bias_equals_tiled(gpu):
    """The linear layer's bias in the persistent kernel's output step (bf16 in and out)."""
    m, n, k = 8192, 2048, 1024
    w = workloads.weight(n, k, seed=72)
    x = workloads.act_normal_bf16(m, k, seed=73).to(gpu)
    bias = torch.from_numpy(np.random.default_rng(74).standard_normal(n).astype(np.float32)).to(torch.bfloat16).to(gpu)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    announce("linear persistent vs tiled", m, n, k)
    outs = {}
    for sched in ("persistent", "tiled"):
        bfp8.set_schedule(sched)
        try:
            outs[sched] = bfp8.linear(x, wq, ws, bias)
            torch.cuda.synchronize()
        finally:
            bfp8.set_schedule("auto")
    assert torch.equal(outs["persistent"].view(torch.int16), outs["tiled"].view(torch.int16))
