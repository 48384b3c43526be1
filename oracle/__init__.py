"""Plain fp64 CPU oracle for exact attention: forward, split-K decode, backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.

Sources (web pages, cited by title and section):

* [xuesongtap] "FlashAttention" (xuesongtap.github.io, 2026-03-22):
  section 1 (definition), 2.1 (tiling), 2.2 (online softmax, the U-update
  equation), 3 (LSE saved for the backward).
* [cnblogs] FlashAttention tiling and distributed article (cnblogs.com,
  jzssuanfa): section 2 (the 4-token worked example), section 3 scenario B
  (FlashDecoding split-K with a pairwise reduction).
* [FA1-vs-FA2] "FlashAttention 1 和 FlashAttention 2 的区别"
  (iceferryling.github.io): section 6 (merging partial (m, l, O) states),
  section 13 (decode is KV-cache bound; paged block tables).
* [operatorworld] "FlashAttention tiling" (operatorworld.com): the online
  softmax update equations and degeneration checks; backward by recomputation.
* [Triton-ch8] "8. FlashAttention 实战" (triton-tutorial.pages.dev):
  section 8.1 (naive attention), 8.3 (online softmax), 8.8 (backward),
  8.9 (FP8 attention: block quantisation, P requantised to FP8,
  incoherent processing).

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against values or properties the pages and the
mathematics fix (worked example, closed forms, finite differences, an
independent autograd implementation).  None is "parity unpinned".
"""

from .attention_ref import (  # noqa: F401
    ref_fwd,
    ref_probs,
    ref_bwd,
    ref_blockwise_fwd,
    online_softmax_step,
    ref_decode_partials,
    merge_two,
    merge_partials_tree,
    ref_splitk_decode,
    decode_chunk_bounds,
    gather_paged_rows,
    ref_paged_decode,
    e4m3_round,
    fp8_block_scale,
    hadamard_rotate,
    quantize_fp8_blocks,
    ref_fwd_fp8,
    ref_merge_lse,
)
