"""GPU-pool residency: lookup, evict, allocate, recall, priority (oracle; test infrastructure only).

ECHO page §5.1 fixes the metadata: a free bitmap over GPU slots
(GPUTokenFree), an eviction priority per slot where low goes first and a free
slot holds -1 (GPUTokenPriority), a fixed-length result buffer with -1 for
invalid entries (GPUIndicesBuffer), and the two maps GPU slot -> host index
(GPUTokenToHost) and host index -> GPU slot (HostTokenToGPU), both holding
infinity when empty.  Its footprint is 4*N_H + 13*N_G bytes.

ECHO page §5.2 describes the three operations.  Allocate: threads holding a
free slot take ranks from an atomic counter and the ranks below the request
size win.  Free: raise the priority of the slots this step selected
(protection), take the lowest-priority slots, and scatter them free in the
bitmap and both maps; no data moves (§2: the host already holds a copy).
Recall: look the selected host indices up in HostTokenToGPU, free + allocate
slots for the misses, update both maps, copy the rows from host memory.

Readings where the page is silent or leaves several results correct:

* infinity = INT32_MAX; the free bitmap is one byte per slot.
* Selected tokens are visited in (request ascending, token ascending) order;
  the misses M keep that order.
* Protection: every slot that holds a selected token is protected this step.
* Eviction happens only when the free slots do not cover the misses: evict
  need = |M| - #free unprotected occupied slots, those with the smallest
  (priority, slot index).  Too few candidates -> status EXHAUSTED and the
  pool is left untouched.  With a reserve R > 0 (room for the next step's
  prefetch, which only takes free slots), the step evicts as many more of the
  same order as it takes to leave R slots free after the allocation, as far
  as unprotected occupied slots allow: need = min(max(0, |M| + R - #free),
  #candidates); only |M| - #free > #candidates is EXHAUSTED.
* Allocation order: the atomic-rank result depends on thread timing, so
  several results are correct.  The canonical rule used for parity: the i-th
  miss takes the i-th free slot in ascending slot order (after eviction).
  `allocate_with_ranks` replays the atomic rule for a given rank order.
* Priority is an integer step stamp (the page calls the policy LRU-like):
  allocated and selected slots get step_id; free slots hold -1.
* GPUIndicesBuffer after a step: entry i holds the slot given to miss i;
  the following entries up to min(N_G, n_rows*k) hold -1; later entries
  are left as they were.
* Errors (status bits): BAD_HOST (a selected host index outside [0, N_H)),
  EXHAUSTED; on either the pool is left untouched.  DUP_HOST (two selected
  misses share a host index) breaks the caller's precondition that requests
  own disjoint host slots; the pool state after it is unspecified.

Pinned by the page's allocate worked example (§5.2), the footprint formula
(§5.1), brute-force eviction on tiny pools, the invariant checker, and
planted-mistake tests proving the checker catches each kind of corruption.
"""

from dataclasses import dataclass

import numpy as np

INF = np.int32(2**31 - 1)
ST_EXHAUSTED = 1
ST_BAD_HOST = 2
ST_DUP_HOST = 4

ROW_ELEMS = 576          # MLA latent row: 512 compressed + 64 RoPE values, bf16 bits


class PoolInvariantError(AssertionError):
    pass


@dataclass
class PoolState:
    free: np.ndarray          # uint8  [N_G]   1 = free
    priority: np.ndarray      # int32  [N_G]   -1 = free
    to_host: np.ndarray       # int32  [N_G]   INF = empty
    host_to_gpu: np.ndarray   # int32  [N_H]   INF = not resident
    indices_buf: np.ndarray   # int32  [N_G]   -1 = invalid
    gpu_kv: np.ndarray        # uint16 [N_G, 576]

    @property
    def n_gpu(self):
        return self.free.shape[0]

    @property
    def n_host(self):
        return self.host_to_gpu.shape[0]

    def copy(self):
        return PoolState(self.free.copy(), self.priority.copy(), self.to_host.copy(),
                         self.host_to_gpu.copy(), self.indices_buf.copy(), self.gpu_kv.copy())

    @staticmethod
    def empty(n_gpu, n_host, poison=0xFFFF):
        return PoolState(np.ones(n_gpu, np.uint8), np.full(n_gpu, -1, np.int32),
                         np.full(n_gpu, INF, np.int32), np.full(n_host, INF, np.int32),
                         np.full(n_gpu, -1, np.int32),
                         np.full((n_gpu, ROW_ELEMS), poison, np.uint16))


@dataclass
class PoolStepResult:
    topk_slot: np.ndarray     # int32 [n_rows, k]; -1 where idx is -1
    miss_host: np.ndarray     # int32 [n_rows*k]; misses in order, -1 after
    miss_slot: np.ndarray     # int32 [n_rows*k]
    n_miss: int
    n_evicted: int
    status: int


def metadata_bytes(n_host, n_gpu):
    """Bytes of pool metadata implied by the dtypes above (§5.1: 4*N_H + 13*N_G)."""
    s = PoolState.empty(1, 1)
    per_slot = (s.free.itemsize + s.priority.itemsize + s.to_host.itemsize
                + s.indices_buf.itemsize)
    return s.host_to_gpu.itemsize * n_host + per_slot * n_gpu


def _selected(sel_idx, key_begin, req_to_host):
    """(row, col, host index) of every selected entry in (row, token) order."""
    rows, cols = np.nonzero(np.asarray(sel_idx) >= 0)      # row-major = (row, token) order
    tok = np.asarray(key_begin, np.int64)[rows] + np.asarray(sel_idx, np.int64)[rows, cols]
    hosts = np.asarray(req_to_host, np.int64)[tok]
    return rows.astype(np.int64), cols.astype(np.int64), hosts


def pool_step(state, host_kv, sel_idx, key_begin, req_to_host, step_id, reserve=0):
    """One guaranteed-residency step for the selected tokens.

    state is not modified; returns (new_state, PoolStepResult).
    sel_idx: int [n_rows, k] token indices per request (-1 = none);
    key_begin[r]: offset of request r in req_to_host; req_to_host: int [n_k]
    host index of every cached token; host_kv: uint16 [N_H, 576]; reserve:
    free slots to leave after the allocation (see the module notes).
    """
    n_rows, k = sel_idx.shape
    n_list = n_rows * k
    out_slot = np.full((n_rows, k), -1, np.int32)
    miss_host = np.full(n_list, -1, np.int32)
    miss_slot = np.full(n_list, -1, np.int32)
    rows, cols, hosts = _selected(sel_idx, key_begin, req_to_host)

    # 1. validate host indices
    if ((hosts < 0) | (hosts >= state.n_host)).any():
        return state, PoolStepResult(out_slot, miss_host, miss_slot, 0, 0, ST_BAD_HOST)

    # 2. lookup: HostTokenToGPU, infinity = miss
    slot_of = state.host_to_gpu[hosts].astype(np.int64)
    hit = slot_of != INF
    miss_pos = np.flatnonzero(~hit)                     # misses in (row, token) order
    m_hosts = hosts[miss_pos]
    n_miss = len(miss_pos)
    miss_host[:n_miss] = m_hosts
    if len(np.unique(m_hosts)) != n_miss:
        return state, PoolStepResult(out_slot, miss_host, miss_slot, n_miss, 0, ST_DUP_HOST)

    # 3. free (evict) only what the misses need beyond the free slots
    protected = np.zeros(state.n_gpu, bool)
    protected[slot_of[hit]] = True
    n_free = int((state.free == 1).sum())
    cand = np.flatnonzero((state.free == 0) & ~protected)
    if max(0, n_miss - n_free) > len(cand):
        return state, PoolStepResult(out_slot, miss_host, miss_slot, n_miss, 0, ST_EXHAUSTED)
    need = min(max(0, n_miss + int(reserve) - n_free), len(cand))
    new = state.copy()
    # smallest (priority, slot): lexsort keys, last key is primary
    evict = cand[np.lexsort((cand, state.priority[cand]))[:need]]
    new.host_to_gpu[new.to_host[evict]] = INF
    new.to_host[evict] = INF
    new.free[evict] = 1
    new.priority[evict] = -1                           # rows stay as they were

    # 4. allocate: i-th miss -> i-th free slot in ascending slot order
    free_slots = np.flatnonzero(new.free == 1)[:n_miss]
    new.free[free_slots] = 0
    new.to_host[free_slots] = m_hosts
    new.host_to_gpu[m_hosts] = free_slots
    new.priority[free_slots] = step_id
    n_buf = min(state.n_gpu, n_list)
    new.indices_buf[:n_buf] = -1
    new.indices_buf[:n_miss] = free_slots
    miss_slot[:n_miss] = free_slots
    slot_of[miss_pos] = free_slots

    # 5. recall: bitwise row copy from the host backup
    new.gpu_kv[free_slots] = host_kv[m_hosts]

    # 6. priority of every selected slot <- this step's stamp
    new.priority[slot_of] = step_id

    out_slot[rows, cols] = slot_of
    return new, PoolStepResult(out_slot, miss_host, miss_slot, n_miss, need, 0)


def allocate_with_ranks(free, ranks, host_indices):
    """Replay of the page's atomic allocate (§5.2) for a given rank order.

    free: bitmap; ranks[t]: the value thread t's atomicAdd returned (only
    threads holding a free slot take one; others pass -1).  Threads whose rank
    is below len(host_indices) win; the winner of rank i is paired with
    host_indices[i].  Returns the allocated slots in rank order.
    """
    size = len(host_indices)
    slots = [-1] * size
    for t, r in enumerate(ranks):
        if free[t] == 1 and 0 <= r < size:
            slots[r] = t
    return slots


def check_pool_invariants(state, host_kv=None, sel_hosts=None, sel_slots=None,
                          protected_before=None, evicted_rows_before=None):
    """Raise PoolInvariantError unless the pool state is consistent.

    Always: free/priority/maps agree on which slots are empty; the two maps
    are mutually inverse on occupied slots (so no slot or host index is
    allocated twice).  Optional: each selected host index sits in the slot
    reported for it with its row equal to the host row bitwise; protected
    slots were not evicted; rows of slots that received no recall are
    unchanged (eviction moves no data).
    """
    free, pri, to_host, h2g = state.free, state.priority, state.to_host, state.host_to_gpu
    if not np.isin(free, (0, 1)).all():
        raise PoolInvariantError("free bitmap holds a value other than 0/1")
    is_free = free == 1
    if not ((to_host == INF) == is_free).all():
        raise PoolInvariantError("free bitmap and GPUTokenToHost disagree")
    if not ((pri == -1) == is_free).all():
        raise PoolInvariantError("free bitmap and priority sentinel disagree")
    occ = np.flatnonzero(~is_free)
    th = to_host[occ].astype(np.int64)
    if ((th < 0) | (th >= state.n_host)).any():
        raise PoolInvariantError("GPUTokenToHost points outside the host pool")
    if len(np.unique(th)) != len(th):
        raise PoolInvariantError("two GPU slots hold the same host index")
    if not (h2g[th] == occ).all():
        raise PoolInvariantError("HostTokenToGPU is not the inverse of GPUTokenToHost")
    resident = np.flatnonzero(h2g != INF)
    if len(resident) != len(occ):
        raise PoolInvariantError("HostTokenToGPU has entries with no owning slot")
    if sel_hosts is not None:
        sel_hosts = np.asarray(sel_hosts, np.int64)
        sel_slots = np.asarray(sel_slots, np.int64)
        if (sel_slots < 0).any():
            raise PoolInvariantError("a selected token has no GPU slot")
        if not (to_host[sel_slots] == sel_hosts).all():
            raise PoolInvariantError("a selected token's slot holds another host index")
        if host_kv is not None and not np.array_equal(state.gpu_kv[sel_slots], host_kv[sel_hosts]):
            raise PoolInvariantError("a selected row differs from its host backup")
    if protected_before is not None:
        p = np.asarray(protected_before, np.int64)
        if (is_free[p]).any():
            raise PoolInvariantError("a protected slot was evicted")
    if evicted_rows_before is not None:
        # (slots, rows before the step) of every slot that received no recall
        slots, rows = evicted_rows_before
        if not np.array_equal(state.gpu_kv[slots], rows):
            raise PoolInvariantError("a row changed in a slot that received no recall")
