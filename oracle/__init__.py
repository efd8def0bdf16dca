"""CPU oracle (test infrastructure only; see oracle/sparsevila.py)."""
from .sparsevila import (  # noqa: F401
    to_f64, retrieval_scores, topk_ascending, retrieve,
    sparse_decode_attn, dense_decode_attn, pack_selected, salience, salience_prune,
    summary_salience, summary_salience_prune, prefill_attention,
)
