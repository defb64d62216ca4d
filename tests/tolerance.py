"""GEMM acceptance against the oracle (tests only).

Bounds (per output element, ref = the oracle's bf16 result, got = the kernel's):
  * mean |got - ref| / mean |ref| <= 1e-3 over the compared elements: the metric
    of the vLLM test on page "prhub.com.cn ... vllm/pull/49932" (section with the
    test source, rel_diff < 0.001);
  * |got - ref| <= 2 ulp_bf16(ref) + 1e-3 |ref| + floor, where
    floor = (K/128 + 130) * 2**-24 * mag and
    mag = sum_kb |As Bs| * sum_k |a_k b_k| (the size of every product entering the
    sum). The first two terms are the stated per-element bound; the floor is the
    worst-case error of float32 accumulation in any order (at most one rounding
    per product-sum step inside a 128-wide block, one for the scale product and
    one per block promotion), which only matters where the sum cancels to near
    zero and 1e-3 |ref| gives no room.

Hardware block dot (only for inputs spread over the whole e4m3 range): the gfx950
FP8 matrix-core instruction does not add its 128 products like IEEE float32. A
product about 13 binades or more below the block's largest product is dropped
(measured: 32 + 2**-9 returns 32). Its error per 128-wide block is thus at most
128 * 2**-13 * max_k |a_k b_k| (times |As Bs|). Tests whose codes are drawn
uniformly over all e4m3 values (magnitudes spread over 36 binades) add
    HW_BLOCK_ETA * mmax,  mmax = sum_kb |As Bs| * max_{k in kb} |a_k b_k|.
The workloads of the pages (uniform activations quantized per group, normal
activations, uniform weights) keep every product of a block within a few binades
of the largest and are held to the bound without this term.
"""

from __future__ import annotations

import numpy as np

from oracle import bf16, e4m3, gemm


def abs_product_mass(a_q, a_s, b_q, b_s, rows, cols):
    """mag[r, c] = sum_kb |As[r,kb] Bs[c//128,kb]| * sum_{k in kb} |a[r,k]| |b[c,k]| (float64)."""
    a_val = np.abs(e4m3.decode(np.asarray(a_q)[rows]))
    b_val = np.abs(e4m3.decode(np.asarray(b_q)[cols]))
    a_sc = np.abs(np.asarray(a_s, np.float64)[rows])
    b_sc = np.abs(np.asarray(b_s, np.float64)[np.asarray(cols) // 128])
    k = a_val.shape[1]
    mag = np.zeros((len(rows), len(cols)))
    for kb in range(-(-k // 128)):  # the last block may be partial
        ks = slice(kb * 128, min(k, kb * 128 + 128))
        mag += (a_val[:, ks] @ b_val[:, ks].T) * (a_sc[:, kb][:, None] * b_sc[:, kb][None, :])
    return mag


HW_BLOCK_ETA = 128 * 2.0**-13


def block_max_mass(a_q, a_s, b_q, b_s, rows, cols):
    """mmax[r, c] = sum_kb |As Bs| * max_{k in kb} |a[r,k]| |b[c,k]| (float64; small shapes only)."""
    a_val = np.abs(e4m3.decode(np.asarray(a_q)[rows]))
    b_val = np.abs(e4m3.decode(np.asarray(b_q)[cols]))
    a_sc = np.abs(np.asarray(a_s, np.float64)[rows])
    b_sc = np.abs(np.asarray(b_s, np.float64)[np.asarray(cols) // 128])
    out = np.zeros((len(rows), len(cols)))
    k_all = a_val.shape[1]
    for kb in range(-(-k_all // 128)):
        cur = np.zeros_like(out)
        for k in range(kb * 128, min(k_all, kb * 128 + 128)):
            np.maximum(cur, np.outer(a_val[:, k], b_val[:, k]), out=cur)
        out += cur * (a_sc[:, kb][:, None] * b_sc[:, kb][None, :])
    return out


def reference(a_q, a_s, b_q, b_s, rows=None, cols=None):
    """(rows, cols, ref_bits, mag) from the oracle."""
    m, n = np.asarray(a_q).shape[0], np.asarray(b_q).shape[0]
    rows = np.arange(m) if rows is None else np.asarray(rows)
    cols = np.arange(n) if cols is None else np.asarray(cols)
    acc, _ = gemm.gemm_acc_ref(a_q, a_s, b_q, b_s, rows, cols)
    mag = abs_product_mass(a_q, a_s, b_q, b_s, rows, cols)
    return rows, cols, bf16.to_bits(acc), mag


def compare(got_bits, ref_bits, mag, k, what="", hw_block=None):
    """Assert the bounds above; returns a dict of statistics. `hw_block` is mmax for tests
    whose codes span the whole e4m3 range (adds HW_BLOCK_ETA * mmax)."""
    got = bf16.from_bits(got_bits)
    ref = bf16.from_bits(ref_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    rel_mean = d.mean() / max(np.abs(ref).mean(), 1e-300)
    stated = 2 * bf16.ulp(ref) + 1e-3 * np.abs(ref)
    floor = (k / 128 + 130) * 2.0**-24 * mag
    if hw_block is not None:
        floor = floor + HW_BLOCK_ETA * hw_block
    bad = d > stated + floor
    stats = {
        "rel_mean": float(rel_mean),
        "max_abs": float(d.max()) if d.size else 0.0,
        "exact_frac": float(np.mean(got_bits == ref_bits)) if d.size else 1.0,
        "over_stated": int((d > stated).sum()),
        "n": int(d.size),
    }
    assert rel_mean <= 1e-3, f"{what}: mean relative error {rel_mean:.3e} > 1e-3 ({stats})"
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements over the bound, first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} ({stats})")
    return stats


def compare_linear(got_bits, ref_out_bits, ref_c_bits, mag, k, what=""):
    """Linear layer: out = bf16(bf16(C) + bias). The GEMM's bound applies to C (at ref_c);
    the bias addition then rounds once more, adding at most one bf16 ulp of the output."""
    got = bf16.from_bits(got_bits)
    ref = bf16.from_bits(ref_out_bits)
    ref_c = bf16.from_bits(ref_c_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    bound = 2 * bf16.ulp(ref_c) + 1e-3 * np.abs(ref_c) + (k / 128 + 130) * 2.0**-24 * mag + bf16.ulp(ref)
    rel_mean = d.mean() / max(np.abs(ref).mean(), 1e-300)
    assert rel_mean <= 1e-3, f"{what}: mean relative error {rel_mean:.3e} > 1e-3"
    bad = d > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements over the bound, first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")
    return {"rel_mean": float(rel_mean), "exact_frac": float(np.mean(got_bits == ref_out_bits))}


# UE8M0 GEMMs: the scaled MFMA adds each K block's product to the running FP32 tile inside
# the matrix core. Measured with one-wave probes (workload-like codes, the running value from
# equal to 4096x the block's mass): error <= 2**-19 * (|running value| + block mass) per step.
# With a 4x margin and |running value| <= mag, K/128 steps give at most
#   (K/128 + 1) * 2**-17 * mag,
# which replaces the float32-accumulation floor of the float-scale path.
E8_STEP_ETA = 2.0**-17


def compare_e8(got_bits, ref_bits, mag, k, what="", hw_block=None):
    """compare() for the UE8M0 GEMMs: the stated bound plus the hardware accumulation floor."""
    got = bf16.from_bits(got_bits)
    ref = bf16.from_bits(ref_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    rel_mean = d.mean() / max(np.abs(ref).mean(), 1e-300)
    stated = 2 * bf16.ulp(ref) + 1e-3 * np.abs(ref)
    floor = (k / 128 + 1) * E8_STEP_ETA * mag
    if hw_block is not None:
        floor = floor + HW_BLOCK_ETA * hw_block
    assert rel_mean <= 1e-3, f"{what}: mean relative error {rel_mean:.3e} > 1e-3"
    bad = d > stated + floor
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {d.size} elements over the bound, first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {(stated + floor)[i]!r}")
    return {"rel_mean": float(rel_mean), "exact_frac": float(np.mean(got_bits == ref_bits)) if d.size else 1.0,
            "over_stated": int((d > stated).sum()), "n": int(d.size)}


def reference_e8(a_q, a_e, b_q, b_e, rows=None, cols=None):
    """(rows, cols, ref_bits, mag) from the oracle, UE8M0 scale codes."""
    from oracle import ue8m0

    return reference(a_q, ue8m0.decode(np.asarray(a_e)).astype(np.float32), b_q,
                     ue8m0.decode(np.asarray(b_e)).astype(np.float32), rows, cols)


def compare_f16(got_bits, ref_bits, mag, k, what=""):
    """compare() for fp16 outputs: the same bound with fp16's ulp (rounded once, to nearest even)."""
    from oracle import f16

    got = f16.from_bits(got_bits)
    ref = f16.from_bits(ref_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    rel_mean = d.mean() / max(np.abs(ref).mean(), 1e-300)
    assert rel_mean <= 1e-3, f"{what}: mean relative error {rel_mean:.3e} > 1e-3"
    bound = 2 * f16.ulp(ref) + 1e-3 * np.abs(ref) + (k / 128 + 130) * 2.0**-24 * mag
    bad = d > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements over the bound, first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")
    return {"rel_mean": float(rel_mean), "exact_frac": float(np.mean(got_bits == ref_bits))}
