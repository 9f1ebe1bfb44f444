"""Lightning-indexer scores (oracle; test infrastructure only).

ECHO page §2 (DSA indexer): for a query token t and a cached token s the
index score is a sum over the H_index = 64 indexer heads of the head weight
w[h,t] times ReLU of the head's query q[h,t] against the token's single
indexer key k[s] (MQA-like: one 128-wide key per token shared by all heads).

Readings where the page is open or garbled:

* The printed formula separates q and k by a comma inside ReLU; the
  "MQA-like" description and the d_index = 128 shapes make it a dot product
  over the 128 dimensions: ReLU(q[h,t] . k[s]).
* Per-token k scale (synthetic general-FP8 workloads): it dequantises k,
  k_deq[s] = scale[s] * k_fp8[s], applied before the ReLU.  Because scale > 0
  this equals applying it after the head sum; the GPU may use either.
* q carries no scale.

Arithmetic: float64.  The per-head dot product of two FP8 vectors is exact in
float64 (each product has <= 8 significant bits with exponents in
[2^-18, 2^17.6], so a 128-term sum needs < 53 bits), whatever order the
library matmul adds in.  The head sum is rounded in float64 (relative error
~1e-16, far below any tolerance used).

Pinned by closed forms (one-hot weights, q = -k, q = k, all-positive inputs
where ReLU is the identity and the score is a plain matrix-vector product),
homogeneity in w and in the k scale, head-permutation invariance, and the
integer-grid exactness argument.
"""

import numpy as np

from .fp8 import decode_e4m3fn


def _request_keys(k, k_scale, begin, length, absolute=False):
    """Decoded (float64) key rows of one request and their scales (None = 1)."""
    kr = decode_e4m3fn(k[begin:begin + length])
    if absolute:
        kr = np.abs(kr)
    sc = None if k_scale is None else np.asarray(k_scale[begin:begin + length], dtype=np.float64)
    return kr, sc


def index_scores(q, w, k, k_scale, key_begin, key_len):
    """Scores of every (query r, key s < key_len[r]) pair.

    q: uint8 [n_q, H, D] E4M3FN; w: float32 [n_q, H]; k: uint8 [n_k, D] E4M3FN;
    k_scale: float32 [n_k] or None; key_begin: int [n_q]; key_len: int [n_q].
    Returns a list of float64 arrays, one per query, of length key_len[r].
    """
    q_dec = decode_e4m3fn(q)                       # [n_q, H, D]
    w64 = np.asarray(w, dtype=np.float64)          # [n_q, H]
    out = []
    for r in range(q_dec.shape[0]):
        kr, sc = _request_keys(k, k_scale, int(key_begin[r]), int(key_len[r]))
        dots = kr @ q_dec[r].T                     # [L, H]: q[h] . k[s], exact
        if sc is not None:
            dots = dots * sc[:, None]              # dequantised key
        out.append(np.maximum(dots, 0.0) @ w64[r])  # sum_h w[h] * ReLU(.)
    return out


def error_scale(q, w, k, k_scale, key_begin, key_len):
    """T[r,s] = scale[s] * sum_h |w[r,h]| * sum_d |q[r,h,d] * k[s,d]|.

    The magnitude of all terms entering score[r,s]; tolerances on general FP8
    inputs are stated relative to it (|gpu - oracle| <= 1e-4 * T).
    """
    q_abs = np.abs(decode_e4m3fn(q))
    w_abs = np.abs(np.asarray(w, dtype=np.float64))
    out = []
    for r in range(q_abs.shape[0]):
        kr, sc = _request_keys(k, k_scale, int(key_begin[r]), int(key_len[r]), absolute=True)
        t = (kr @ q_abs[r].T) @ w_abs[r]
        if sc is not None:
            t = t * sc
        out.append(t)
    return out


def prefill_scores_rows(q, w, k, rows, k_scale=None):
    """Causal prefill scores for the query rows listed in `rows`.

    The prefill indexer scores every (query t, key s <= t) pair (ECHO page
    §3.4: the indexer is quadratic in the context).  Reading of "causal
    mask": keys s <= t, the diagonal included.  q: [T, H, D], k: [T, D].
    Returns a list of float64 arrays, row t having length t + 1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    k_dec = decode_e4m3fn(k)                       # [T, D], decoded once for every row
    sc = None if k_scale is None else np.asarray(k_scale, dtype=np.float64)
    q_dec = decode_e4m3fn(q[rows])                 # [rows, H, D]
    w64 = np.asarray(w, dtype=np.float64)[rows]
    out = []
    for i, t in enumerate(rows):
        dots = k_dec[:t + 1] @ q_dec[i].T          # [t+1, H]: q[h] . k[s], exact
        if sc is not None:
            dots = dots * sc[:t + 1, None]
        out.append(np.maximum(dots, 0.0) @ w64[i])
    return out
