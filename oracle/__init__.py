"""CPU oracle for the NVFP4 W4A4 and MXFP8 W8A8 linear-layer hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it. It shares no code, table or constant
generator with the HIP library; it is written from the format definitions and
from what the pages state the operations compute:

* FastVideo nvfp4_config.py page: the ``_nvfp4_quantize`` / ``_mm_fp4``
  wrappers and their shape (fake) kernels; NVFP4 = e2m1 values, one e4m3
  scale per 16 elements, an fp32 alpha and the ``layout_128x4`` scale layout.
* FastVideo nvfp4_qat_config.py page: ``convert_model_to_fp4`` (weight global
  scale 448*6/amax) and ``NVFP4QATQuantizeMethod.apply`` (static activation
  global scale 1.0, alpha = 1/(x_gsf*w_gsf)).
* SGLang nvfp4_online.py page: ``_quantize_weight_nvfp4`` (amax == 0 guard,
  K % 16 check, e4m3 max from the float8_e4m3fn format).
* vLLM-Omni mxfp8_config.py page: ``DiffusionMXFP8Config`` (32-element groups
  along K sharing one e8m0 scale, per the OCP MX spec) and the online
  BF16 -> MXFP8 weight conversion.
* The bias each page's linear method adds after the GEMM (``linear``).
* The norm whose fused quantize may hand mm_fp4 a ``pre_quantized`` triple
  (FastVideo nvfp4_config.py, ``NVFP4QuantizeMethod.apply``): RMSNorm (``norm``).

Floating-point steps are carried out in IEEE fp32 with numpy float32 arithmetic
(every operation rounded to nearest even, no fused multiply-add), because the
quantizer's outputs are integers decided by fp32 arithmetic; GEMM references
are fp64. Where the pages leave a step open, the reading taken is stated at the
function that implements it.

Pinning: every function here is checked in ``tests/test_oracle_*.py`` against
values fixed by the format definitions and hand-worked examples
(``tests/golden/``), closed forms, invariants and brute force; none is
"parity unpinned" except where a function docstring says so.
"""
from . import activations, formats, linear, mxfp4, mxfp8, norm, nvfp4  # noqa: F401
