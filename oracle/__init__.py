"""Plain, slow CPU oracle for the DSA-indexer + top-k + pool-residency decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package; only the test-suite, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP library: it works on
numpy arrays in float64, with library primitives (matmul, sort) used only as
single steps of the definition.

Citations name the web page and the section on it:

* "ECHO page" = the blog review "OSDI'26 | ECHO：稀疏 attention 省了算力，
  却把 HBM 撑爆了" (marsggbo.github.io, 2026-07-29), sections numbered as on
  that page (§2 concepts, §5.1 metadata, §5.2 in-graph operations, §6.1
  intra-query prefetching, §6.2 inter-query prefetching, §6.3 the indexer
  kernel with a copy stage).

Modules: fp8 (E4M3FN decoding), scores (indexer scores and their error
scale), topk (exact top-k, sample threshold), pool (the residency step),
decode (one whole step), multistep (steps in a row: new tokens with
write-through, the EMA threshold), interquery (the chunked prefill's
approximate top-k subsets under the shifted histogram, and its unions),
prefetch (what the page fixes about the threshold prefetch: the eligible
tokens, the bound in proportion to the context, the contract a prefetched pool
satisfies, and one valid outcome).

Readings of points the page leaves open are listed in each module's docstring.
Parity status of every function is stated in its docstring ("pinned by ...").
"""

from .fp8 import E4M3FN_TABLE, decode_e4m3fn
from .scores import index_scores, error_scale, prefill_scores_rows
from .topk import topk_row, topk_rows, sample_threshold, threshold_bin
from .pool import (INF, ST_EXHAUSTED, ST_BAD_HOST, ST_DUP_HOST, PoolState,
                   pool_step, allocate_with_ranks, metadata_bytes,
                   check_pool_invariants, PoolInvariantError)
from .decode import decode_step
from .multistep import (KeyCache, ST_CACHE_FULL, append_tokens, kth_scores, ema_update,
                        decode_loop)
from .interquery import approx_subset, union_segments, prefill_chunk_loop
from .prefetch import (prefetch_eligible, prefetch_bound, apply_prefetch, greedy_prefetch,
                       check_prefetch_contract)

__all__ = [
    "E4M3FN_TABLE", "decode_e4m3fn", "index_scores", "error_scale",
    "prefill_scores_rows", "topk_row", "topk_rows", "sample_threshold",
    "threshold_bin", "INF", "ST_EXHAUSTED", "ST_BAD_HOST", "ST_DUP_HOST",
    "PoolState", "pool_step", "allocate_with_ranks", "metadata_bytes",
    "check_pool_invariants", "PoolInvariantError", "decode_step", "KeyCache",
    "ST_CACHE_FULL", "append_tokens", "kth_scores", "ema_update", "decode_loop",
    "approx_subset", "union_segments", "prefill_chunk_loop", "prefetch_eligible",
    "prefetch_bound", "apply_prefetch", "greedy_prefetch", "check_prefetch_contract",
]
