"""CPU oracle for exact scaled-dot-product attention — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this package imports nothing
from the product path: the two share no code.

Everything here is plain float64 numpy (or pure-Python floats) written to be
checked against the pages by eye, not to be fast.  Pages cited (title, address):

  [A100]  "告别OOM和训练慢：用Flash Attention加速你的PyTorch大模型（含A100环境配置）"
          http://www.cyqw.cn/news/1153354
  [PT29]  "PyTorch-CUDA-v2.9镜像中使用FlashAttention提升训练速度"
          http://www.yongjin360.com/news/212413
  [FA37]  "Flash Attention 3.7 核心原理与实战：加速Transformer模型训练与推理"
          http://www.hmyw.cn/news/56989
  [VRAM]  "显存神技：必学FlashAttention！"
          https://gitcode.csdn.net/69e6287b0a2f6a37c5a11aee.html

Modules
  attention  the definition: materialise S and P per (batch, head) in float64
             (forward, backward, row-sampled forward) — pinned
  brute      a scalar pure-Python evaluation of the unshifted softmax formula,
             used only to pin ``attention`` on tiny shapes — pinned (by the
             closed forms and by ``attention``)
  online     the tiled running-max / running-sum recurrence in the pages'
             order — pinned against ``attention``
  padded     padded batches (per-sample lengths) and packed ones (sequences concatenated
             per head, offsets): the definition over each
             sample's own rows, zeros past them — pinned
  cross      N_q queries over N_k keys, the queries being the last N_q positions
             (decode steps, a new block over a cache), optional ALiBi distance
             penalty and block-sparse mask, forward and backward — pinned
  dropout    attention dropout with masks from Philox4x32-10 (a published
             counter-based generator), forward and backward — pinned
  fp8        decode steps over an FP8 (E4M3) key/value cache, and the forward over
             FP8 queries, keys and values: the code values from the OCP definition,
             then ``cross`` / ``attention`` over the descaled values — pinned
  pool       a process pool over (batch, head) for timing the oracle on a
             bounded sample

Every function has at least one pin in ``tests/test_oracle*.py`` that does not
re-type its formula; no function is "parity unpinned".
"""
from .attention import (allowed_mask, attention_forward, attention_backward,
                        attention_forward_rows, attention_forward_bh, attention_backward_bh,
                        allowed_pairs, score_matrix_nbytes)
from .online import attention_forward_online
from .brute import attention_forward_brute
from .padded import (clamp_lengths, packed_backward, packed_forward, packed_ranges,
                     padded_backward_bh, padded_forward_bh)
from .cross import (BLOCK, alibi_bias, block_allowed, cross_allowed_mask, cross_allowed_pairs, cross_backward,
                    cross_backward_bh, cross_forward, cross_forward_bh)

from .dropout import (dropout_backward, dropout_backward_bh, dropout_forward, dropout_forward_bh,
                      dropout_keep, keep_scale, keep_threshold, philox4x32_10)
from .fp8 import e4m3_value, fp8_cache_forward, fp8_cache_forward_bh, fp8_forward

__all__ = [
    "allowed_mask", "attention_forward", "attention_backward", "attention_forward_rows",
    "attention_forward_bh", "attention_backward_bh", "allowed_pairs", "score_matrix_nbytes",
    "attention_forward_online", "attention_forward_brute",
    "clamp_lengths", "padded_forward_bh", "padded_backward_bh", "packed_ranges",
    "packed_forward", "packed_backward",
    "cross_allowed_mask", "cross_allowed_pairs", "cross_forward", "cross_forward_bh",
    "cross_backward", "cross_backward_bh", "alibi_bias", "BLOCK", "block_allowed",
    "philox4x32_10", "keep_threshold", "keep_scale", "dropout_keep", "dropout_forward", "dropout_backward",
    "dropout_forward_bh", "dropout_backward_bh",
    "e4m3_value", "fp8_cache_forward", "fp8_cache_forward_bh", "fp8_forward",
]
