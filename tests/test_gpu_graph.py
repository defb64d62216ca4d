"""The library's launches captured in a HIP graph replay to the eager results (quantizer, every
GEMM schedule including the persistent override, the one-launch and two-launch linear layer, the
no-allocation linear, the 1x64 layout and the whole experts chain), replay after replay, with
eager work and synchronizations in between."""

import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [9, 256, 2048])
def test_graph_replays_match_eager(gpu, m):
    w = workloads.weight(1024, 2048, seed=41)
    x = workloads.act_uniform(m, 2048, seed=42).to(gpu)
    bq, bs = w.q.to(gpu), w.s.to(gpu)
    q = torch.empty(m, 2048, dtype=torch.uint8, device=gpu)
    s = torch.empty(16, m, dtype=torch.float32, device=gpu).t()
    c = torch.empty(m, 1024, dtype=torch.bfloat16, device=gpu)
    announce("graph capture", m)

    def run():
        bfp8.quant_act(x, q=q, scales=s)
        bfp8.gemm(q, s, bq, bs, out=c)

    run()
    torch.cuda.synchronize()
    q_ref, s_ref, c_ref = q.clone(), s.clone(), c.clone()

    side = torch.cuda.Stream(gpu)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        q.fill_(0)
        c.fill_(0)
        s.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_ref), f"replay {rep}: codes differ"
        assert torch.equal(s, s_ref), f"replay {rep}: scales differ"
        assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16)), f"replay {rep}: GEMM output differs"
        run()  # eager work between replays
        torch.cuda.synchronize()


def _replays_match_eager(gpu, run, outs, what):
    """Run eagerly, capture run() on a side stream, then replay four times (outputs cleared
    before each replay, eager runs and synchronizations between replays): every replay must
    reproduce the eager outputs bit for bit."""
    run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    side = torch.cuda.Stream(gpu)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run()
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o.contiguous().view(torch.uint8), r.contiguous().view(torch.uint8)), \
                f"{what}: replay {rep}, output {i} differs"
        run()
        torch.cuda.synchronize()


# M = 1 and 4 take the one-launch path (quantizer fused into the K-split GEMM), M = 64 the
# quantizer and the GEMM as two launches; the bias is added in the epilogue.
@pytest.mark.parametrize("m", [1, 4, 64])
def test_graph_linear(gpu, m):
    n, k = 2048, 5120
    w = workloads.weight(n, k, seed=43)
    x = workloads.act_normal_bf16(m, k, seed=44).to(gpu)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    bias = workloads.act_normal_bf16(1, n, seed=45)[0].to(gpu)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=gpu)
    ws_buf = torch.empty(bfp8.linear_workspace_bytes(m, n, k), dtype=torch.uint8, device=gpu)
    announce("graph linear", m, n, k, "one launch" if bfp8.linear_fuses(m, n, k) else "two launches")
    assert bfp8.linear_fuses(m, n, k) == (m <= 4)
    _replays_match_eager(gpu, lambda: bfp8.linear(x, wq, ws, bias=bias, out=out, workspace=ws_buf), [out],
                         f"linear M={m}")


@pytest.mark.parametrize("m", [3, 300])
def test_graph_linear_noalloc(gpu, m):
    n, k = 1024, 4096
    w = workloads.weight(n, k, seed=46)
    x = workloads.act_normal_bf16(m, k, seed=47).to(gpu)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=gpu)
    announce("graph linear_noalloc", m, n, k)
    _replays_match_eager(gpu, lambda: bfp8.linear_noalloc(x, wq, ws, out), [out], f"linear_noalloc M={m}")


# K-split (M = 16, and M = 1000 on 1024 columns), then the tiled kernel on 128 x 128 tiles
# (M = 1000, 4096 columns) and on 256 x 256 tiles (M = 4096), all with a K tail.
@pytest.mark.parametrize("m,n", [(16, 1024), (1000, 1024), (1000, 4096), (4096, 4096)])
def test_graph_1x64(gpu, m, n):
    k = 4160
    w = workloads.weight_1x64(n, k, seed=48)
    x = workloads.act_uniform(m, k, seed=49).to(gpu)
    wq, ws = bfp8.pad_k(w.q.to(gpu)), w.s.to(gpu)
    q, s = bfp8.quant_act_1x64(x)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=gpu)
    announce("graph 1x64", m, n, k)

    def run():
        q2, s2 = bfp8.quant_act_1x64(x)
        q.copy_(q2)
        s.copy_(s2)
        bfp8.gemm_1x64(q, s, wq, ws, out=c)

    _replays_match_eager(gpu, run, [q, s, c], f"1x64 M={m}")


def test_graph_persistent_schedule(gpu):
    m, n, k = 8448, 2048, 128  # two tiles of 256 x 256 per workgroup
    w = workloads.weight(n, k, seed=50)
    x = workloads.act_uniform(m, k, seed=51).to(gpu)
    wq, ws = w.q.to(gpu), w.s.to(gpu)
    q, s = bfp8.quant_act(x)
    c = torch.empty(m, n, dtype=torch.bfloat16, device=gpu)
    announce("graph persistent", m, n, k)
    bfp8.set_schedule("persistent")
    try:
        _replays_match_eager(gpu, lambda: bfp8.gemm(q, s, wq, ws, out=c), [c], "persistent schedule")
    finally:
        bfp8.set_schedule("auto")


def test_graph_moe_forward(gpu):
    """The whole experts chain (dispatch, gathered quantization, two grouped GEMMs, SwiGLU +
    quantization, combine) as one graph: every grid is sized on the host from the token count,
    nothing is read back."""
    t, k, e, h, i = 96, 8, 16, 1024, 512
    x = workloads.act_normal_bf16(t, h, seed=52).to(gpu)
    ids, wts = workloads.moe_routing(t, k, e, seed=53)
    ids, wts = ids.to(gpu), wts.to(gpu)
    wu, su, wdn, sdn = (a.to(gpu) for a in workloads.moe_experts(e, h, i, seed=54))
    out = torch.empty(t, h, dtype=torch.bfloat16, device=gpu)
    ws_buf = torch.empty(bfp8.moe_forward_workspace_bytes(t, k, e, h, i), dtype=torch.uint8, device=gpu)
    announce("graph moe_forward", t, k, e, h, i)
    _replays_match_eager(gpu, lambda: bfp8.moe_forward(x, ids, wts, wu, su, wdn, sdn, out=out, workspace=ws_buf),
                         [out], "moe_forward")
