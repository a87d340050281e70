"""CPU fp64 oracle for fused exact attention -- TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  The HIP library under ``exact_attention_17_amd`` never
imports it, links it or falls back to it, and this package imports nothing
from there: the two share no code.  Seeded inputs come from ``workloads``,
which holds no attention arithmetic.

What it computes is the plain definition of attention, with the score matrix
S and the probability matrix P materialised in float64:

    S = scale * Q K^T  (+ mask as -inf),  P = softmax(S) row-wise,  O = P V,
    LSE = m + ln(l) per query row.

Sources (pages on the subject, cited by title and section):
  * "FlashAttention-3 vs naive attention: inference comparison (FA3)",
    sec. 1.1 -- the standard definition S, P, O and the 5-step naive pipeline.
  * "FlashAttention" concept page, sec. "Definition" -- softmax(QK^T/sqrt(d_k))V.
  * "FIA / FlashAttention" explainer, sec. 1 -- online softmax keeps a running
    row max m and normaliser l and reproduces the global softmax exactly.
  * "flash-attention" configuration skill page, sec. 3.2-3.5 and appendix
    (PagedAttention, FlashDecoding / Split-KV, GQA/MQA, continuous batching)
    -- argument shapes, causal / window_size, cu_seqlens, block_table, GQA,
    and k_new / v_new appended to a KV cache of cache_seqlens tokens.

Readings where the pages are silent:
  causal alignment is bottom-right; window bounds are inclusive; -1 means an
  unbounded window side; query head h uses KV head h // (Hq // Hkv); LSE is the
  natural-log log-sum-exp of the scaled scores; a row with no visible key has
  O = 0 and LSE = -inf; new K/V rows are appended at positions
  cache_seqlens[b] + i; softcap acts on the scaled logits and the ALiBi bias,
  -slope * |i + Lk - Lq - j|, is added after it, both before the mask.

Gradients (``backward.py``): the derivative of that definition for an
upstream gradient dO, by the chain rule -- dV = P^T dO, dS = P * (dO V^T - D)
with D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q, summed over the
query heads of a KV group.  The pages fix only that a fused backward
recomputes the blocks from saved row statistics ("FlashAttention" concept
page, recomputation; "FIA / FlashAttention" explainer, sec. 1); the values
are those of the plain definition.

Inputs are numpy arrays; a uint16 array is taken as bfloat16 bit patterns
(numpy has no bfloat16 type) and converted exactly to float64.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_backward_pins.py`` against closed forms, invariants, a
pure-Python brute force, central finite differences, PyTorch's CPU
``scaled_dot_product_attention`` and autograd in float64.  No function is
parity-unpinned.
"""

from .attention import (
    key_visibility,
    attend_rows,
    alibi_bias,
    attention_ref,
    attention_rows_ref,
    attention_varlen_ref,
    gather_paged,
    decode_paged_ref,
    append_paged_ref,
    attention_kvcache_ref,
    decode_split_partials_ref,
    merge_partials_ref,
    online_softmax_ref,
)
from .backward import (
    attention_bwd_rows,
    attention_bwd_ref,
    attention_bwd_query_rows_ref,
    attention_bwd_key_rows_ref,
    attention_varlen_bwd_ref,
)

__all__ = [
    "key_visibility",
    "attend_rows",
    "alibi_bias",
    "attention_ref",
    "attention_rows_ref",
    "attention_varlen_ref",
    "gather_paged",
    "decode_paged_ref",
    "append_paged_ref",
    "attention_kvcache_ref",
    "decode_split_partials_ref",
    "merge_partials_ref",
    "online_softmax_ref",
    "attention_bwd_rows",
    "attention_bwd_ref",
    "attention_bwd_query_rows_ref",
    "attention_bwd_key_rows_ref",
    "attention_varlen_bwd_ref",
]
