"""Plain fp64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library or its Python binding, and imports neither.

What it computes (each function cites the page passage it follows):

* ``attention``      -- softmax(scale * Q K^T) V, materialising S and P in fp64,
                        with causal / block / key-length masks and GQA heads.
* ``decode``         -- one new query per sequence against a KV cache.
* ``logit_bound``    -- the Cauchy-Schwarz upper bound on each row's logits
                        (optionally with mean-centred keys).
* ``fixed_max_bounds`` -- the per-row bound over the keys a row can see,
                        its gap to the row max and the eligibility rule.
* ``round_to_bf16``   -- round to the nearest bfloat16 (ties to even).
* ``fixed_max_attention`` -- softmax evaluated against the bound instead of the
                        row maximum (equal to ``attention`` in exact arithmetic).
* ``online_softmax``  -- the running (max, sum) recurrence over blocks of a row.
* ``merge_partials``  -- combining (O, LSE) pairs of disjoint key sets.
* ``attention_backward`` -- dQ, dK, dV of the same function for an upstream
                        gradient dO (chain rule through S, P and the softmax).

Pins (tests/test_oracle.py): printed worked examples (tests/golden/), closed
forms (single key, identical keys, causal first row), invariants (row sums,
joint permutation, shift invariance, split == unsplit), library routines
(torch SDPA in float64 on the CPU, scipy logsumexp) and an independent
frame-gather construction for block masks. The gradients are pinned to
central finite differences of the forward oracle, to closed forms (constant V,
a single key), to invariants (key-shift invariance, value-gradient sums) and to
torch autograd in float64 on the CPU (tests/test_oracle_backward.py).

Parity unpinned: the eligibility threshold ``TAU`` = 64 is a constant chosen
here from an underflow argument, not a value the pages give; only the rule's
soundness (the normaliser stays far above the fp32 minimum) is tested. The
same holds for ``MIN_KEYS`` = 64, the fewest visible keys for which a row
takes the fixed max.
"""

from .backward import attention_backward  # noqa: F401
from .attention import (  # noqa: F401
    MIN_KEYS,
    TAU,
    attention,
    decode,
    element_mask,
    fixed_max_attention,
    fixed_max_bounds,
    logit_bound,
    merge_partials,
    online_softmax,
    round_to_bf16,
)
