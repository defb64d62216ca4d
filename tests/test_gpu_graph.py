"""The library's launches captured in a HIP graph replay to the eager results (quantizer and
every GEMM schedule), replay after replay, with eager work and synchronizations in between."""

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
