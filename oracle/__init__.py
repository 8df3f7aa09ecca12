"""CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 reference
that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The library under ``exact_attention_flash_amd/`` never imports it,
and it imports nothing from that library: the two share no code.

Sources (the web pages this method is described on):

* "优化的注意力实现 (FlashAttention)" (apxml course page), section
  "标准注意力中的内存带宽瓶颈": the definition softmax(Q K^T / sqrt(d_k)) V;
  its PyTorch example gives the manual fallback procedure (scale, additive
  causal bias from ``tril(diagonal=0)`` filled with -inf, row softmax, @ V).
* "Transformer、注意力机制与优化" (CMU 15-442/642 notes), section "数学公式"
  (the same definition, Q, K, V in R^{N x d}) and section
  "安全 Softmax 与在线 Softmax" (m(x), f(x), l(x) and the two-block merge).
* "FlashAttention 的基本原理", section 2.4 "反向传播": dV from P^T dO and the
  per-row softmax gradient; the same notes' section
  "为什么前向和反向的并行化策略不同" give dQ_i += dS^(j) K_j.
* "FlashAttention 系列技术详解", FlashAttention-3 section: FP8 matrix
  products.  ``fp8`` decodes OCP E4M3 inputs (format from the OCP 8-bit
  floating point specification) and runs the same exact attention on them.
* "FlashAttention 的基本原理", section 2.4 (the backward algorithm also covers
  dropout) and the apxml example (dropout on the attention weights):
  ``dropout`` draws the keep mask with Philox4x32-10 (Salmon et al., SC 2011)
  and gives the forward and the gradients with the mask applied.

Every function names the passage it follows.  All arithmetic is float64.

Pins: every function here is pinned by ``tests/test_oracle_*.py`` to
something other than itself (a hand-derived worked example, brute force on
tiny inputs, closed forms, library special cases, finite differences,
invariants).  No function is "parity unpinned".
"""

from .attention import (
    widen_bf16,
    scores,
    softmax_rows,
    softmax_row_grad,
    attention_probs,
    attention_forward,
    attention_forward_rows,
    attention_backward,
    attention_backward_sampled,
)
from .fp8 import (
    decode_e4m3,
    dequantize,
    attention_forward_fp8,
    attention_forward_fp8_rows,
    hadamard_matrix,
    incoherent_rotation,
    encode_e4m3,
    quantize_e4m3,
)
from .dropout import (
    philox,
    dropout_threshold,
    dropout_scale,
    dropout_bytes,
    dropout_mask,
    attention_forward_dropout,
    attention_forward_dropout_rows,
    attention_backward_dropout,
    attention_backward_dropout_head,
)
from .online_softmax import (
    softmax_stats,
    merge_stats,
    fold_blocks,
    blockwise_forward_head,
)

__all__ = [
    "widen_bf16",
    "scores",
    "softmax_rows",
    "softmax_row_grad",
    "attention_probs",
    "attention_forward",
    "attention_forward_rows",
    "attention_backward",
    "attention_backward_sampled",
    "decode_e4m3",
    "dequantize",
    "attention_forward_fp8",
    "attention_forward_fp8_rows",
    "hadamard_matrix",
    "incoherent_rotation",
    "encode_e4m3",
    "quantize_e4m3",
    "philox",
    "dropout_threshold",
    "dropout_scale",
    "dropout_bytes",
    "dropout_mask",
    "attention_forward_dropout",
    "attention_forward_dropout_rows",
    "attention_backward_dropout",
    "attention_backward_dropout_head",
    "softmax_stats",
    "merge_stats",
    "fold_blocks",
    "blockwise_forward_head",
]
