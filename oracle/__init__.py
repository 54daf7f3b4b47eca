"""CPU oracle for the causal video tokenizer hot path (test infrastructure only).

This package is the slow, plain, obviously-correct reference that the HIP
library is checked against.  It is test infrastructure: only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it.  The product
path (the HIP library and its Python binding) never imports, calls or links it,
and it shares no code with that path.

All floating-point arithmetic is float64 (NumPy); bf16 inputs are decoded
exactly and bf16 outputs are re-encoded by the oracle's own round-to-nearest-
even encoder (``oracle.bf16``).

Sources (the web pages describing the Cosmos Tokenizer):

* "NVIDIA Cosmos Tokenizer 完全指南：图像与视频神经分词器（Neural Tokenizer）的原理、
  安装与推理实战" (a walkthrough of the tokenizer README), sections 6.1, 6.2,
  7.1 (Haar wavelet patching), 7.2 (FSQ) and 7.3 (causal design).
* "nvidia/Cosmos-Tokenize1-CV8x8x8-720p" (model card), section
  "Model Architecture".
* "Cosmos World Foundation Model Platform for Physical AI (Cosmos-Predict1)"
  (paper summary), section "1) Cosmos Tokenizer" (factorized convolution and
  factorized causal self-attention).
* FSQ's bound function follows the published method: Mentzer et al. 2023,
  "Finite Scalar Quantization: VQ-VAE Made Simple" (arXiv:2309.15505).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force or library routines.  No function is
"parity unpinned"; the free conventions the pages leave open (channel order,
high-pass sign, FSQ epsilon) are documented where they are fixed.
"""

from . import bf16, haar, conv, fsq, attention  # noqa: F401
