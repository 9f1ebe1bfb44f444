"""Seeded synthetic inputs for the decode step and the prefill indexer.

This module only draws numbers: it holds none of the method's arithmetic, and
both the CPU oracle and the HIP library receive what it produces.  Every
array comes from numpy's PCG64 seeded by (seed, array tag), so an array does
not depend on the order others are drawn in.

Workloads (the synthetic stand-ins for the long-context serving traces the
ECHO page measures with; real traces and model weights are not used):

  tiny      1 request x 4096 tokens, integer-grid q/k, k=256, pool = half of
            all tokens (random), full
  b8_64k    8 x 65536, integer-grid, k=2048, 90% of selected resident, pool
            = N_H/8, full
  b32_ragged 32 x U[16384,131072], general FP8 with per-token k scale,
            k=2048, 70% of selected resident, host pool 8x GPU pool, full
  prefill_32k  causal 32768 x 32768, integer grid, per-row top-2048
  b64_128k  64 x 131072, general FP8 with k scale, k=2048, 50% of selected
            resident, 131072 free slots kept for prefetch
  multi-step loops (make_multistep_inputs): B requests of a given length run
            several decode steps; every step draws a new query and one new
            token per request (key, key scale, latent row, a fresh host row)

Value recipes:
  integer grid: q, k uniform integers in [-8, 8] (exact in E4M3FN);
                w uniform integers in [-4, 4] / 64
  general:      q, k ~ N(0,1) rounded to E4M3FN (nearest even);
                w ~ N(0,1)/8; k scale ~ U[0.5, 2]
  latent rows:  576 bf16 bit patterns per token, uniform random bits (PCG64 raw
                output) with bit 14 cleared (finite, |x| < 2, never the 0xFFFF
                poison pattern);
                the recall copies bits, so their distribution is immaterial
  host slots:   the tokens of all requests occupy a seeded permutation of
                the host pool
  pool state:   a given fraction of each request's selected tokens is made
                resident at random, the rest of the pool is filled with
                random unselected tokens, occupied slots take distinct
                random priorities from a permutation of [0, N_G) and the
                step stamp is N_G; free slots hold the poison pattern
  paged keys:   a request's keys copied into fixed-size pages handed out in a
                seeded random order (page_key_cache)
"""

from dataclasses import dataclass, field
import math

import numpy as np

H_INDEX = 64
D_INDEX = 128
ROW_ELEMS = 576
POISON = 0xFFFF
INF = 2**31 - 1

_TAGS = {"q": 1, "w": 2, "k": 3, "scale": 4, "len": 5, "perm": 6, "kv": 7,
         "hit": 8, "fill": 9, "slots": 10, "prio": 11, "scores": 12, "step": 13, "pages": 14}


def rng_for(seed, tag):
    return np.random.default_rng([int(seed), _TAGS[tag]])


@dataclass
class DecodeConfig:
    name: str
    batch: int
    lengths: object            # int, or (lo, hi) for uniform per-request lengths
    topk: int
    grid: str                  # "int" or "general"
    k_scale: bool
    hit_rate: float            # fraction of selected tokens resident before the step
    pool_div: int              # N_G = ceil(N_H / pool_div)
    reserve: int = 0           # free slots kept empty (prefetch room)
    resident_of_all: bool = False   # tiny: residency drawn over all tokens
    prefetch: bool = False
    seed: int = 1


CONFIGS = {
    "tiny": DecodeConfig("tiny", 1, 4096, 256, "int", False, 0.5, 2, seed=1,
                         resident_of_all=True),
    "b8_64k": DecodeConfig("b8_64k", 8, 65536, 2048, "int", False, 0.9, 8, seed=2),
    "b32_ragged": DecodeConfig("b32_ragged", 32, (16384, 131072), 2048, "general", True,
                               0.7, 8, seed=3),
    "b64_128k": DecodeConfig("b64_128k", 64, 131072, 2048, "general", True, 0.5, 8,
                             reserve=131072, prefetch=True, seed=5),
}

PREFILL = {"prefill_32k": dict(n=32768, topk=2048, grid="int", seed=4)}


def _int_to_e4m3_table():
    import torch
    vals = torch.arange(-8, 9, dtype=torch.float32)
    return vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def e4m3_from_f32(x):
    """Round float32 values to E4M3FN bytes (nearest even) with torch's conversion."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_values(seed, tag, shape, grid, chunk=1 << 24, workers=None):
    """uint8 E4M3FN array of the given shape, integer-grid or N(0,1).

    Drawn in chunks of `chunk` values, chunk c from PCG64 seeded by (seed, tag, c), so the
    content does not depend on the number of worker threads.
    """
    import concurrent.futures as cf
    import os
    n = int(np.prod(shape))
    out = np.empty(n, np.uint8)
    table = _int_to_e4m3_table() if grid == "int" else None

    def one(c):
        s = c * chunk
        m = min(chunk, n - s)
        rng = np.random.default_rng([int(seed), _TAGS[tag], c])
        if grid == "int":
            out[s:s + m] = table[rng.integers(0, 17, m, dtype=np.int8)]
        else:
            out[s:s + m] = e4m3_from_f32(rng.standard_normal(m, dtype=np.float32))

    n_chunks = (n + chunk - 1) // chunk
    workers = workers or min(16, os.cpu_count() or 1)
    if n_chunks <= 1 or workers <= 1:
        for c in range(n_chunks):
            one(c)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(n_chunks)))
    return out.reshape(shape)


def head_weights(seed, n, grid):
    rng = rng_for(seed, "w")
    if grid == "int":
        return (rng.integers(-4, 5, (n, H_INDEX)).astype(np.float32) / np.float32(64.0))
    return (rng.standard_normal((n, H_INDEX), dtype=np.float32) / np.float32(8.0))


def request_lengths(cfg):
    if isinstance(cfg.lengths, (tuple, list)):
        lo, hi = cfg.lengths
        return rng_for(cfg.seed, "len").integers(lo, hi + 1, cfg.batch).astype(np.int32)
    return np.full(cfg.batch, int(cfg.lengths), np.int32)


def fill_latent_rows(seed, out, chunk_rows=1 << 16, workers=None):
    """Fill a uint16 [N, 576] array (may be pinned host memory) in place.

    Rows are drawn in chunks of `chunk_rows`, chunk c from PCG64 seeded by (seed, tag, c), so
    the content does not depend on the number of worker threads.
    """
    import concurrent.futures as cf
    import os
    n = out.shape[0]
    flat = out.reshape(n, ROW_ELEMS)

    def one(c):
        s = c * chunk_rows
        m = min(chunk_rows, n - s)
        bg = np.random.default_rng([int(seed), _TAGS["kv"], c]).bit_generator
        raw = bg.random_raw(m * ROW_ELEMS // 4).view(np.uint16).reshape(m, ROW_ELEMS)
        np.bitwise_and(raw, np.uint16(0xBFFF), out=flat[s:s + m])

    n_chunks = (n + chunk_rows - 1) // chunk_rows
    workers = workers or min(16, os.cpu_count() or 1)
    if n_chunks <= 1 or workers <= 1:
        for c in range(n_chunks):
            one(c)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(n_chunks)))
    return out


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q: np.ndarray            # uint8 [B, 64, 128]
    w: np.ndarray            # float32 [B, 64]
    k: np.ndarray            # uint8 [sum L, 128]
    k_scale: object          # float32 [sum L] or None
    key_begin: np.ndarray    # int64 [B]
    key_len: np.ndarray      # int32 [B]
    req_to_host: np.ndarray  # int32 [sum L]
    n_host: int
    n_gpu: int
    extra: dict = field(default_factory=dict)


def make_decode_inputs(cfg, lengths=None):
    """Draw q, w, k, k scale and the token -> host-slot map for a config."""
    key_len = request_lengths(cfg) if lengths is None else np.asarray(lengths, np.int32)
    key_begin = np.zeros(len(key_len), np.int64)
    key_begin[1:] = np.cumsum(key_len.astype(np.int64))[:-1]
    n_tok = int(key_len.astype(np.int64).sum())
    q = fp8_values(cfg.seed, "q", (len(key_len), H_INDEX, D_INDEX), cfg.grid)
    w = head_weights(cfg.seed, len(key_len), cfg.grid)
    k = fp8_values(cfg.seed, "k", (n_tok, D_INDEX), cfg.grid)
    k_scale = None
    if cfg.k_scale:
        k_scale = rng_for(cfg.seed, "scale").uniform(0.5, 2.0, n_tok).astype(np.float32)
    req_to_host = rng_for(cfg.seed, "perm").permutation(n_tok).astype(np.int32)
    n_host = n_tok
    n_gpu = int(math.ceil(n_host / cfg.pool_div))
    return DecodeInputs(cfg, q, w, k, k_scale, key_begin, key_len, req_to_host, n_host, n_gpu)


@dataclass
class PoolArrays:
    free: np.ndarray
    priority: np.ndarray
    to_host: np.ndarray
    host_to_gpu: np.ndarray
    indices_buf: np.ndarray
    gpu_kv: np.ndarray
    step_id: int


def make_pool_state(inp, selected, host_kv, hit_rate=None, reserve=None):
    """Initial pool for one step.

    selected: int [B, k] token indices per request (-1 padded), the set the
    step will select; a `hit_rate` fraction of each request's selected tokens
    is made resident, the remaining capacity (minus `reserve` free slots) is
    filled with random unselected tokens.  For the tiny workload the resident
    set is a random half of all tokens instead.
    """
    cfg = inp.cfg
    hit_rate = cfg.hit_rate if hit_rate is None else hit_rate
    reserve = cfg.reserve if reserve is None else reserve
    n_gpu, n_host = inp.n_gpu, inp.n_host
    n_tok = inp.k.shape[0]
    rng_hit, rng_fill = rng_for(cfg.seed, "hit"), rng_for(cfg.seed, "fill")
    capacity = n_gpu - reserve
    if cfg.resident_of_all:
        resident_tok = rng_fill.permutation(n_tok)[:capacity]
    else:
        chosen = []
        is_sel = np.zeros(n_tok, bool)
        for r in range(selected.shape[0]):
            s = selected[r][selected[r] >= 0].astype(np.int64) + int(inp.key_begin[r])
            is_sel[s] = True
            n_hit = int(round(hit_rate * len(s)))
            chosen.append(rng_hit.permutation(s)[:n_hit])
        chosen = np.concatenate(chosen) if chosen else np.zeros(0, np.int64)
        if len(chosen) > capacity:
            raise ValueError("pool too small for the requested hit rate")
        others = np.flatnonzero(~is_sel)
        n_fill = min(capacity - len(chosen), len(others))
        filler = others[rng_fill.choice(len(others), n_fill, replace=False)] if n_fill else others[:0]
        resident_tok = np.concatenate([chosen, filler])
    hosts = inp.req_to_host[resident_tok].astype(np.int64)
    slots = rng_for(cfg.seed, "slots").permutation(n_gpu)[:len(hosts)]
    free = np.ones(n_gpu, np.uint8)
    priority = np.full(n_gpu, -1, np.int32)
    to_host = np.full(n_gpu, INF, np.int32)
    host_to_gpu = np.full(n_host, INF, np.int32)
    free[slots] = 0
    to_host[slots] = hosts
    host_to_gpu[hosts] = slots
    priority[slots] = rng_for(cfg.seed, "prio").permutation(n_gpu)[:len(slots)]
    gpu_kv = np.full((n_gpu, ROW_ELEMS), POISON, np.uint16)
    gpu_kv[slots] = host_kv[hosts]
    return PoolArrays(free, priority, to_host, host_to_gpu,
                      np.full(n_gpu, -1, np.int32), gpu_kv, step_id=n_gpu)


def random_scores(seed, n_rows, length, tie_frac=0.0, ld=None):
    """float32 score rows for the top-k alone, with optional planted ties."""
    rng = rng_for(seed, "scores")
    ld = length if ld is None else ld
    s = rng.standard_normal((n_rows, ld), dtype=np.float32)
    if tie_frac > 0:
        m = rng.random((n_rows, ld)) < tie_frac
        s[m] = np.round(s[m] * 4) / 4          # coarse grid -> many equal values
    return s


def make_prefill_inputs(n, grid="int", seed=4):
    q = fp8_values(seed, "q", (n, H_INDEX, D_INDEX), grid)
    w = head_weights(seed, n, grid)
    k = fp8_values(seed, "k", (n, D_INDEX), grid)
    return q, w, k


@dataclass
class MultiStepInputs:
    k: np.ndarray            # uint8 [B * capacity, 128]; rows past key_len are zero
    k_scale: object          # float32 [B * capacity] or None
    key_begin: np.ndarray    # int64 [B]: r * capacity
    key_len: np.ndarray      # int32 [B]: initial lengths
    req_to_host: np.ndarray  # int32 [B * capacity]; rows past key_len hold -1
    capacity: int
    n_host: int
    n_gpu: int
    pool: PoolArrays         # initial pool; step stamps start at pool.step_id
    steps: list              # dicts: q, w, new_k, new_scale, new_kv, new_host, step_id


def make_multistep_inputs(batch, length, n_steps, n_gpu, grid="int", k_scale=False, seed=11,
                          reserve=0, drift=None):
    """A loop of n_steps decode steps over `batch` requests that start with `length` tokens.

    Host rows: the initial tokens occupy a seeded permutation of [0, batch*length), the new
    tokens a seeded permutation of the following batch*n_steps rows.  The pool starts full but
    for `reserve` free slots (random tokens resident, distinct random priorities from a
    permutation of
    [0, n_gpu)); step stamps are n_gpu, n_gpu + 1, ...  Latent rows of the initial tokens come
    from fill_latent_rows(seed, ...); the host rows of the new tokens hold the poison pattern
    until their token is appended, and the new tokens' own rows come from
    fill_latent_rows(seed + 7919, ...).  Queries: independent draws per step, or with
    `drift` = f the first step's q and w carried on with a fraction f of q's bytes redrawn each
    step (consecutive decode queries of a request are alike, so their selections overlap).
    Returns (MultiStepInputs, host_kv)."""
    cap = length + n_steps
    n0 = batch * length
    n_host = n0 + batch * n_steps
    cfg = DecodeConfig("multistep", batch, length, 0, grid, k_scale, 0.0, 1, seed=seed)
    base = make_decode_inputs(cfg)
    key_begin = np.arange(batch, dtype=np.int64) * cap
    k = np.zeros((batch * cap, D_INDEX), np.uint8)
    req_to_host = np.full(batch * cap, -1, np.int32)
    ks = np.zeros(batch * cap, np.float32) if k_scale else None
    for r in range(batch):
        src = slice(r * length, (r + 1) * length)
        dst = slice(r * cap, r * cap + length)
        k[dst] = base.k[src]
        req_to_host[dst] = base.req_to_host[src]
        if k_scale:
            ks[dst] = base.k_scale[src]
    host_kv = fill_latent_rows(seed, np.empty((n_host, ROW_ELEMS), np.uint16))
    host_kv[n0:] = POISON                      # rows of tokens not generated yet
    new_kv = fill_latent_rows(seed + 7919, np.empty((batch * n_steps, ROW_ELEMS), np.uint16))
    # initial pool: random resident tokens, all slots used
    n_res = min(n_gpu - reserve, n0)
    tok = rng_for(seed, "fill").permutation(n0)[:n_res]
    hosts = base.req_to_host[tok].astype(np.int64)
    slots = rng_for(seed, "slots").permutation(n_gpu)[:n_res]
    free = np.ones(n_gpu, np.uint8)
    priority = np.full(n_gpu, -1, np.int32)
    to_host = np.full(n_gpu, INF, np.int32)
    host_to_gpu = np.full(n_host, INF, np.int32)
    free[slots] = 0
    to_host[slots] = hosts
    host_to_gpu[hosts] = slots
    priority[slots] = rng_for(seed, "prio").permutation(n_gpu)[:n_res]
    gpu_kv = np.full((n_gpu, ROW_ELEMS), POISON, np.uint16)
    gpu_kv[slots] = host_kv[hosts]
    pool = PoolArrays(free, priority, to_host, host_to_gpu, np.full(n_gpu, -1, np.int32),
                      gpu_kv, step_id=n_gpu)
    new_hosts = (n0 + rng_for(seed, "step").permutation(batch * n_steps)).astype(np.int32)
    steps = []
    q_prev = w0 = None
    for t in range(n_steps):
        s_seed = seed * 1000 + t + 1
        nh = new_hosts[t * batch:(t + 1) * batch]
        q_t = fp8_values(s_seed, "q", (batch, H_INDEX, D_INDEX), grid)
        w_t = head_weights(s_seed, batch, grid)
        if drift is not None:
            if q_prev is None:
                w0 = w_t
            else:
                keep = rng_for(s_seed, "hit").random(q_t.shape) >= drift
                q_t = np.where(keep, q_prev, q_t)
                w_t = w0
            q_prev = q_t
        steps.append(dict(
            q=q_t,
            w=w_t,
            new_k=fp8_values(s_seed, "k", (batch, D_INDEX), grid),
            new_scale=(rng_for(s_seed, "scale").uniform(0.5, 2.0, batch).astype(np.float32)
                       if k_scale else None),
            new_kv=new_kv[t * batch:(t + 1) * batch].copy(),
            new_host=nh.copy(),
            step_id=n_gpu + t))
    return MultiStepInputs(k, ks, key_begin, np.full(batch, length, np.int32), req_to_host,
                           cap, n_host, n_gpu, pool, steps), host_kv


class PagedKeys:
    """A request-contiguous key cache laid out in fixed-size pages: k_pages [n_pages * P, 128]
    (and k_scale_pages [n_pages * P] or None), page_table [n_rows, max_pages] int32 (page ids,
    -1 past a request's last page).  Pages are handed out in a seeded random order, so that a
    request's pages are scattered as in a paged cache that has been allocated from and freed."""

    def __init__(self, k_pages, k_scale_pages, page_table, page_size):
        self.k_pages, self.k_scale_pages = k_pages, k_scale_pages
        self.page_table, self.page_size = page_table, page_size


def page_key_cache(k, k_scale, key_begin, key_len, page_size, seed, spare_pages=3):
    """The keys of `key_begin`/`key_len` (rows of k, k_scale) copied into pages of `page_size`
    tokens; the tail of a request's last page and the spare pages hold random bytes (never
    read).  No arithmetic of the method: a layout change only."""
    rng = rng_for(seed, "pages")
    n_rows = len(key_len)
    per = [-(-int(L) // page_size) for L in key_len]
    max_pages = max(1, max(per) if per else 1)
    n_pages = sum(per) + spare_pages
    order = rng.permutation(n_pages).astype(np.int32)
    k_pages = rng.integers(0, 256, (n_pages * page_size, k.shape[1]), dtype=np.uint8)
    k_pages[(k_pages & 0x7F) == 0x7F] = 0                   # no NaN codes, even where unread
    ks_pages = None
    if k_scale is not None:
        ks_pages = rng.uniform(0.5, 2.0, n_pages * page_size).astype(np.float32)
    table = np.full((n_rows, max_pages), -1, np.int32)
    nxt = 0
    for r in range(n_rows):
        L, b = int(key_len[r]), int(key_begin[r])
        for j in range(per[r]):
            p = int(order[nxt])
            nxt += 1
            table[r, j] = p
            n = min(page_size, L - j * page_size)
            k_pages[p * page_size:p * page_size + n] = k[b + j * page_size:b + j * page_size + n]
            if ks_pages is not None:
                ks_pages[p * page_size:p * page_size + n] = k_scale[b + j * page_size:b + j * page_size + n]
    return PagedKeys(k_pages, ks_pages, table, page_size)
