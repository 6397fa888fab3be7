"""Plain CPU oracle for the 4-bit block-quantized weight matmul.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``bit_quantized_weight_amd/``.

What it computes (NumPy, float64 wherever the pages leave precision open):

* ``q4``  -- the 4-bit block weight format: quantize, pack, unpack,
  dequantize, and the weight-streaming matmul ``Y = X . What^T`` used by
  decode and speculative verification.  Source: "Qwen3.8-27B at 256K on a
  24GB RTX PRO 4000 SFF (432 GB/s): 50 tok/s with MTP" (page 3), the
  paragraphs on weight streaming during autoregressive decode and on the
  public Q4_0 GGUF.  The page names the format but does not define it; the
  definition used is: 32-element blocks along K, an fp16 scale equal to
  absmax/7, signed 4-bit codes, two codes per byte.
* ``a8``  -- the A8 prefill route: int8 activations per token per 64
  channels, exact int32 block sums against the 4-bit weights, fp32-class
  rescale.  Source: "Qwen3.8-27B on RTX 4090: 5,000 tok/s Prefill
  Reproduced" (page 5), section "Why the A8 artifact matters".

* ``attn`` -- the decode-time attention read of a K/V cache held in the same
  4-bit block format: softmax(q . K^T / sqrt(D)) V over the visible cache
  positions, grouped query heads.  Source: page 3, the architecture and
  bandwidth paragraphs (16 full-attention layers with a 4-bit K/V cache
  whose reads grow with the context).

Every reading of an open point is listed in the docstring of the function
that takes it.  Parity pins live in ``tests/test_oracle_*.py``.
"""

from . import q4, a8, attn  # noqa: F401
