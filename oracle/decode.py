"""One whole decode step: scores -> exact top-k -> guaranteed residency (oracle; test infrastructure only).

ECHO page §4 (overall design): the indexer scores every cached token, the
exact top-k picks the tokens sparse attention will read, and a guaranteed
recall makes every picked token's latent row resident in the GPU pool; the
priorities are then refreshed.  Prefetch (§6.1) only moves rows earlier and
never changes the selected set, so the oracle's result is the one without
prefetch; a step with prefetch must produce the same selected set and the
same selected rows.
"""

from .scores import index_scores
from .topk import topk_rows
from .pool import pool_step


def decode_step(q, w, k, k_scale, key_begin, key_len, req_to_host, state, host_kv,
                topk_k, step_id):
    """Returns (scores list[float64], idx int32 [B, k], new_state, PoolStepResult)."""
    scores = index_scores(q, w, k, k_scale, key_begin, key_len)
    idx = topk_rows(scores, topk_k)
    new_state, res = pool_step(state, host_kv, idx, key_begin, req_to_host, step_id)
    return scores, idx, new_state, res
