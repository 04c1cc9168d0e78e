"""Plain fp64 CPU oracle for one GPU's share of a sequence-parallel attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links or
executes this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP library and imports nothing
from it; both sides receive the same seeded arrays from the input generators.

Every function is the plain definition of what the pages describe, written out
in float64 numpy with no blocking, fusion or reordering beyond the definition:

* ``permute``   -- the Ulysses sequence-shard <-> head-shard re-layout
                   (Keryc, "Ulysses SP: entrenar modelos con millones de tokens",
                   section "Como funciona Ulysses Sequence Parallelism (SP)";
                   DeepSpeed-Ulysses notes, section "Method", the all-to-all table).
* ``attention`` -- exact softmax attention with the position_ids document mask,
                   and its analytic gradients (Ultralytics glossary "Ring
                   Attention", section "Como funciona la atencion en anillo";
                   aitoolresearcher Ulysses SP review, section 3, position_ids).
* ``merge``     -- combination of partial (O, LSE) results by the cumulative
                   softmax (Ring Attention page, same section).
* ``ring``      -- the four-device ring simulation of the Ring Attention page,
                   in the page's raw-exp form and in the running-max form.
* ``striped``   -- the striped token layout of the same page's Striped Attention
                   remark (rank r holds tokens r, r + P, ...), attention between
                   two stripes, and the ring over stripes.

Pins (tests/test_oracle_*.py) tie each function to facts the pages and the
mathematics fix; see the test modules for which pin covers which function.
"""

from .permute import seq_to_head, head_to_seq, seq_to_head_elementwise
from .attention import (visible_mask, attention_fwd, attention_bwd,
                        attention_probs, causal_visible_pairs)
from .merge import lse_merge
from .ring import ring_sim_raw, ring_sim_online, full_attention_noncausal
from .striped import seq_to_stripe, stripe_to_seq, striped_pair_fwd, striped_ring_fwd

__all__ = [
    "seq_to_head", "head_to_seq", "seq_to_head_elementwise",
    "visible_mask", "attention_fwd", "attention_bwd", "attention_probs",
    "causal_visible_pairs", "lse_merge",
    "ring_sim_raw", "ring_sim_online", "full_attention_noncausal",
    "seq_to_stripe", "stripe_to_seq", "striped_pair_fwd", "striped_ring_fwd",
]
