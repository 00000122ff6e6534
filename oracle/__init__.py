"""CPU oracle for the group-wise low-bit weight-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain definition of what
the HIP library computes.  Only the test-suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.  The product path (``bit_quantized_linear_int4_amd``) never
imports, links or calls anything here, and this package imports nothing from
the product path: the two share no code, tables or constants.

Everything is NumPy (plus the Python standard library for the normal
quantile function).  Decisions that turn floats into integers (codes, zero
points, outlier flags) are taken in IEEE fp32, the precision the kernels use;
reference matrix products are taken in fp64.

Pages cited (titles translated; the section numbers are the pages' own):

[P1] "大模型量化选型：五种主流方案对比与实战" -- "LLM quantization selection:
     five mainstream schemes compared", www.0539edu.com/news/5934728
[P2] "很多人对量化的理解，只停在‘把模型变小’" -- the quantization-concepts
     article (INT8, INT4, GPTQ, AWQ, SmoothQuant, NF4, QLoRA),
     aicoding.csdn.net/6a6874d110ee7a33f2936327.html
[P3] "LLM量化实操手册" -- "LLM quantization hands-on manual",
     devpress.csdn.net/awstech/6a472a61662f9a54cb88fc6c.html
[P4] "开源模型量化实战指南：GGUF、GPTQ、AWQ选型与本地部署" -- "Open-source model
     quantization guide: GGUF, GPTQ, AWQ selection and local deployment",
     chuanbook.com/?id=280
[P5] "【推理与部署篇05】模型量化部署深度对比：GPTQ、AWQ、GGUF与FP8实战指南" --
     "Inference & deployment 05: quantized deployment compared (GPTQ, AWQ,
     GGUF, FP8)", devpress.csdn.net/amd/6a55d4ea662f9a54cb8f2c4c.html

Modules:
  numerics   -- round-to-nearest-even helpers (fp16, bf16, integer rounding)
  int4       -- asymmetric INT4 group quantization, packing, dequantization
  nf4        -- NF4 codebook, blockwise absmax encode, double quantization
  llm_int8   -- LLM.int8() vector-wise int8 with outlier-column decomposition
  linear     -- the fp64 reference linear y = x . w_hat^T
"""

from . import numerics, int4, nf4, llm_int8, linear  # noqa: F401
