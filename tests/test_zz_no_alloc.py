"""bfp8_linear_noalloc (the linear layer staged in the library's fixed device array, for callers
that cannot allocate) against bfp8_linear on the same inputs, bit for bit: two calls in a row,
the second with a smaller layer, so the second call runs over the staging the first one left."""

import numpy as np
import pytest
import torch

import block_scaled_fp8_bfp8_amd as bfp8
import workloads
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def _case(m, k, n, dtype, with_bias, seed):
    x = workloads.act_normal_bf16(m, k, seed=seed).to(dtype)
    w = workloads.weight(n, k, seed=seed + 1)
    bias = None
    if with_bias:
        bias = torch.from_numpy(np.random.default_rng(seed + 2).standard_normal(n).astype(np.float32)).to(dtype)
    return x, w.q, w.s, bias


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_noalloc_equals_linear_on_two_calls(gpu, dtype):
    # the first layer stages 2048 x 5120 codes; the second a smaller one with a partial last K block
    for m, k, n, with_bias, seed in [(2048, 5120, 1280, True, 700), (37, 1008, 600, False, 710)]:
        x, wq, ws, bias = _case(m, k, n, dtype, with_bias, seed)
        x, wq, ws = x.to(gpu), bfp8.pad_k(wq.to(gpu)), ws.to(gpu)  # weight rows of whole 128-byte blocks
        bias = bias.to(gpu) if bias is not None else None
        announce("linear_noalloc", m, k, n, dtype, with_bias)
        want = bfp8.linear(x, wq, ws, bias)
        out = torch.full((m, n), float("nan"), dtype=dtype, device=gpu)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(gpu)
        bfp8.linear_noalloc(x, wq, ws, out, bias)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(gpu) == before
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"M={m} K={k} N={n}"


def test_noalloc_rejects_staging_beyond_its_array(gpu):
    m, k, n = 2048, 40960, 256  # 84 MB of codes > 64 MiB
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=gpu)
    wq = torch.zeros((n, k), dtype=torch.uint8, device=gpu)
    ws = torch.ones((2, k // 128), dtype=torch.float32, device=gpu)
    out = torch.zeros((m, n), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(NotImplementedError, match="staging"):
        bfp8.linear_noalloc(x, wq, ws, out)
