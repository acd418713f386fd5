"""CPU oracle for the TokenGate pruned-prefill hot path (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""

from .tokengate_oracle import (  # noqa: F401
    LOG2E,
    gate_score,
    gated_layer,
    gather_kept,
    keybias_attention,
    keybias_attention_gate_grads,
    keybias_attention_gate_grads_at,
    keybias_decode,
    kept_counts,
    random_budgets,
    random_k_select,
    random_scores,
    rope,
    silu,
    splitmix64,
    topk_select,
)
