"""MI355X (gfx950) hot path of TokenGate's pruned prefill.

gate score -> top-K select (question always kept) -> compaction -> token-gated
causal GQA attention over the kept tokens, as hand-written HIP kernels behind a
C ABI (include/tokengate.h).  This package is the thin Python binding; the
library is loaded lazily by _lib.load(), and nothing here runs on the CPU.
"""

from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    TokenGateError,
    load,
    tg_attn_decode,
    tg_attn_decode_workspace_bytes,
    tg_attn_forward,
    tg_attn_gate_grads,
    tg_attn_gate_grads_workspace_bytes,
    tg_attn_prepare,
    tg_attn_workspace_bytes,
    tg_gate_score,
    tg_gated_select,
    tg_gather_kept,
    tg_kept_counts,
    tg_keybias_attn_prefill,
    tg_random_budgets,
    tg_random_k_select,
    tg_topk_select,
    tg_topk_workspace_bytes,
)
