"""Helpers for the GPU parity tests (tests only)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import block_scaled_fp8_bfp8_amd as bfp8
from oracle import quant


def announce(*parts) -> None:
    """Name the case before a GPU step, so a fault can be traced to it."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def quant_gpu_checked(x_cpu: torch.Tensor, dev, what: str = ""):
    """Quantize on the GPU and assert bit-exactness against the oracle.

    Returns (q_dev [M,K] uint8, s_dev [M,K/128] group-major, q_ref, s_ref)."""
    announce("quant_act", what, tuple(x_cpu.shape), x_cpu.dtype)
    x = x_cpu.to(dev)
    q, s = bfp8.quant_act(x)
    torch.cuda.synchronize()
    q_ref, s_ref = quant.quant_act_ref(x_cpu.float().numpy())
    q_got = q.cpu().numpy()
    s_got = s.cpu().contiguous().numpy()
    if not np.array_equal(q_got, q_ref):
        idx = np.argwhere(q_got != q_ref)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} q codes differ, first at {i}: got {q_got[i]:#x} "
                             f"want {q_ref[i]:#x} (x = {x_cpu.float().numpy()[i]!r})")
    if not np.array_equal(s_got.view(np.uint32), s_ref.view(np.uint32)):
        idx = np.argwhere(s_got.view(np.uint32) != s_ref.view(np.uint32))
        raise AssertionError(f"{what}: {len(idx)} scales differ, first at {tuple(idx[0])}")
    return q, s, q_ref, s_ref


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (numpy, host)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
