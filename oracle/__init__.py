"""CPU oracle for the fused two-stage MXFP4 mixture-of-experts FFN with the SiTUv2 activation.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
package: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP implementation (no kernels, headers, tables or helpers) and
computes everything in float64 with NumPy, from the definitions on the source pages:

* github ROCm/aiter PR 6259, "Motivation": SiTUv2 (situ(g) = beta*tanh(g/beta)*sigmoid(g),
  up = linear_beta*tanh(u/linear_beta)) and the wide-MoE shape it serves.
* github ROCm/aiter PR 4463, "What" and "Three tuner defects": bf16 / fp8 / fp4x2 activation
  dtypes, fp4x2 packing (two e2m1 codes per byte) and nibble-wise comparison.
* github ROCm/aiter PR 5118, "Summary": the moe_sorting step that groups routed rows by expert
  and pads every expert to a whole block_m.
* github ROCm/aiter PR 4471, "Motivation" / "Technical Details": the SiLU and SiTUv2 stage1
  epilogues y = act(gate) * up.

Modules
-------
mx_formats  e2m1 / e4m3fn / e8m0 decoding and the 1x32 block quantization rule.
moe         routing sort layout, stage1, stage2 and the whole fused operator.

Parity status of every function is stated in its module header.
"""
from . import mx_formats, moe  # noqa: F401
