"""CPU oracle for blockwise-scaled FP8 GEMM (1x128 activation groups, 128x128 weight blocks).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (``block_scaled_fp8_bfp8_amd``) never imports it, and this package
imports nothing from the product path: the two share no code, tables or helpers.

What is computed, and where it is defined on the pages:

* e4m3fn codec (``e4m3``): the OCP float8 e4m3 "fn" format named by the vLLM
  test on page "prhub.com.cn ... vllm/pull/49932" (section "关键源码片段": the
  ``torch.float8_e4m3fn`` dtype and its ``finfo`` max of 448).
* bf16 rounding (``bf16``): the bf16 output dtype of the same test and of the
  ``gemm_fp8_fp8_bf16_nt`` kernel named on page "vllm-project/vllm/pull/19085".
* per-token-group quantizer (``quant``): ``per_token_group_quant_fp8(x, 128)``
  of the vLLM test and ``per_token_cast_to_fp8`` (gran_k=128, fp32 scale
  factors) on page "transformers/integrations/deepgemm.py"
  (``_select_fp8_cast_kwargs``, ``deepgemm_fp8_fp4_linear``).
* blockwise GEMM (``gemm``): C[m,n] = sum_kb (A_q[m,kb] . B_q[n,kb]) * As[m,kb] * Bs[n//128,kb],
  the ``native_w8a8_block_matmul`` reference of the vLLM test, with the
  1x128 / 128x128 block contract of its "实现拆解" list item 2.
* 1x64 / 128x64 layout (``quant.quant_act_ref(x, group=64)``, ``gemm.gemm_acc_ref(...,
  k_block=64)``): the next block-scale layouts named on the vLLM torch-backend page (section
  "风险与影响"), read as the same definitions over 64-wide K groups with 128-row weight blocks.
* M-grouped contiguous GEMM (``gemm.grouped_gemm_contiguous_ref``): page
  "transformers/integrations/deepgemm.py", ``_build_deepgemm_contiguous_layout``
  (per-row expert id, -1 on padding rows) and ``deepgemm_fp8_fp4_experts_forward``.
* fp16 rounding (``f16``): the fp16 output of the linear layer for fp16 activations (same page
  as below: the output dtype follows the input).
* FP8 linear layer (``linear.linear_ref``): page "transformers/integrations/deepgemm.py",
  ``deepgemm_fp8_fp4_linear`` (quantize, GEMM into a bf16 output, then add the bias to it).
* MoE chain (``moe``): same page, ``_dispatch_routed_input``, ``_build_deepgemm_contiguous_layout``,
  ``deepgemm_fp8_fp4_experts_forward`` and ``_combine_routed_output`` (routing layout, the
  expert MLP with the gate activation between the two grouped GEMMs, weighted top-k combine).
* UE8M0 (power-of-two) scale factors (``ue8m0``): same page, ``_ceil_to_ue8m0``,
  ``_select_fp8_cast_kwargs`` (``use_ue8m0``) and ``_coerce_sf_for_kernel``
  (``float8_e8m0fnu`` codes): the quantizer with its scale rounded up to a power of two,
  and the blockwise GEMM of operands carrying such scales.

Every function is pinned by tests under ``tests/test_oracle_*.py`` (library
routines, brute force with exact rationals, closed forms and invariants),
including the spacing helpers ``bf16.ulp``, ``e4m3.ulp`` and ``f16.ulp`` that
set the acceptance bounds (``tests/test_oracle_ulp.py``: the distance to the
next value as torch and numpy decode neighbouring bit patterns); none is
"parity unpinned".
"""

from . import bf16, e4m3, f16, gemm, linear, moe, quant, scales, ue8m0  # noqa: F401

__all__ = ["bf16", "e4m3", "f16", "gemm", "linear", "moe", "quant", "ue8m0"]
