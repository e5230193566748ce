"""Plain fp64 CPU oracle for the paged KV store and paged attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``paged_kv_attention_28_amd``) never imports it and
shares no code with it: no kernels, headers, helpers, constants or pre/post
processing. The only code both sides use is the seeded input generator in
``workloads/``, which holds none of the method's arithmetic.

Sources (cited by page title and section throughout):

* P1 = page "13. 读一个最小推理引擎：nano-vllm" (niuwancheng.cn).
* P2 = page "读 Nano-vLLM 源码：一个极简 LLM 推理引擎是如何工作的" (keriko-blog).

Functions and what pins them (see ``tests/test_oracle.py``):

* ``prepare_step_ref``   per-step metadata (slot mapping etc.).
  Pinned by a hand-derived fixture under ``tests/golden/`` and by invariants.
* ``kv_store_ref``       bit copy of token rows into the paged cache.
  Pinned by row-by-row definitional checks and sentinel-untouched checks.
* ``gather_context_ref`` logical-to-physical gather through a block table.
  Pinned by permutation invariance and paged == contiguous.
* ``attn_contiguous_ref`` masked softmax attention on dense K/V.
  Pinned by closed forms (single key, identical keys, zero query), the convex
  hull property, causality, GQA head tagging, chunked == one-shot, decode ==
  last prefill row, a scalar brute force, and torch's fp64 CPU
  ``scaled_dot_product_attention`` as an independent library routine.
* ``decode_ref`` / ``prefill_ref`` compose the above.

Readings of points the pages leave open (softmax scale 1/sqrt(D), GQA head
mapping h // (H_q / H_kv), bottom-right causal alignment, zero output for
padding rows) are listed in the module docstrings where they are used.
Softmax scale and head mapping are conventions no page value fixes: parity
with the pages is unpinned for those two choices beyond the invariants above.
"""

from .paged import (  # noqa: F401
    bf16_bits_to_f64,
    prepare_step_ref,
    kv_store_ref,
    kv_store_inplace_ref,
    gather_context_ref,
    attn_contiguous_ref,
    decode_ref,
    prefill_ref,
)
