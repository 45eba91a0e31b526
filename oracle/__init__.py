"""CPU fp64 oracle for scaled-dot-product attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it, and
it shares no code with the HIP path (the two meet only in the seeded input
generators of ``workloads``).

What it computes is the plain definition of attention that all three pages
take for granted (flash prefill in "WAVE: A Symbolic Python DSL and Compiler
for High Performance Machine Learning (MLSys 2026)", core method; flash
decoding with a page table in "Wave February 2025 Release", FlashDecoding
list):

    O[b,h,i,:] = sum_j softmax_j(scale * <q_i, k_j> + M_ij) * v_j,
    M_ij = -inf  iff causal and j > i + (Skv - Sq)   (bottom-right aligned),

in float64 from the exact upcast of the fp16/bf16 inputs.  Paged decode is the
same function at Sq = 1 applied to each sequence's keys and values, gathered
explicitly through the page table.  With fewer KV heads than query heads
(grouped-query / multi-query attention, which the pages do not define), query
head h reads KV head h // (H / H_kv).  Extend attention (new tokens after a
cached prefix) is causal attention over the prefix gathered through the page
table followed by the new tokens, bottom-right aligned.  FP8 attention is
the same function of the dequantised inputs (e4m3fn code x per-tensor
descale).  The backward pass is the gradient of sum(O * dO) by the chain rule
(``sdpa_backward``; ``sdpa_backward_dq_rows`` and ``sdpa_backward_kv_rows``
form selected rows of it at full size); ``lse_rows`` is each row's log-sum-exp.

Pinned by ``tests/test_oracle.py`` (brute force at 50 digits, the torch
library routine, closed forms, invariants) and
``tests/test_oracle_mutations.py`` (each planted mistake fails a pin).
"""
from .attention import (  # noqa: F401
    attend_rows,
    attention_probs,
    dequantize_fp8,
    extend,
    gather_sequence,
    kv_head,
    lse_rows,
    sdpa_backward,
    sdpa_backward_dq_rows,
    sdpa_backward_kv_rows,
    n_visible,
    paged_decode,
    sdpa,
    sdpa_rows,
    to_f64,
)
