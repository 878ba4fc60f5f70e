"""CPU oracle for the DeepSeekMoE layer forward (test infrastructure only).

This package is the slow, plain reference that the HIP path is checked
against.  Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import it; the product path never does, and it shares no
code, table or helper with the HIP kernels.

What each module computes, and the passage it follows:

* ``formats``  - OCP E4M3FN encode/decode and bf16 rounding, from the format
  definitions (the pages only say "FP8"; see the readings in the design notes).
* ``quant``    - 1x128 activation tiles and 128x128 weight blocks, from the
  news.qq.com article (news.qq.com/rain/a/20241229A05OQF00), section
  FP8 低精度训练 › 细粒度量化, and the aliyun study note, section 4.1.
* ``route``    - sigmoid scores, per-expert selection bias, group-limited
  top-k, from the aliyun study note section 2.2 and the news.qq.com article
  sections DeepSeekMoE 架构, 无额外损耗的负载均衡 and 节点限制路由.
* ``balance``  - the aux-loss-free bias update, same passages.
* ``permute``  - token dispatch order (the all-to-all dispatch of a DualPipe
  chunk, news.qq.com article section DualPipe 流水线并行).
* ``gemm``     - block-scaled FP8 GEMM with high-precision accumulation,
  news.qq.com article section FP8 低精度训练 › 提高累加精度.
* ``swiglu``   - SwiGLU + requantisation (the pages are silent on the expert
  FFN form; SwiGLU is the workload definition).
* ``combine``  - weighted combine plus the shared expert.
* ``layer``    - the whole forward, and a per-token direct form used as a pin.

Parity pins: every function here is pinned in ``tests/test_oracle_*.py``.
Parity unpinned by the pages: the pages print no worked example, so every
pin is a closed form, an invariant, a brute force or a library cross-check.
"""
from . import formats, quant, route, balance, permute, gemm, swiglu, combine, layer  # noqa: F401
