"""The stress decode workload at full size (64 requests x 131072 tokens, general FP8 keys with
per-token scales, top-2048, half of the selection resident in a pool of 2^20 slots with 131072
kept free, threshold prefetch from a 4096-score sample, the step captured as one hipGraph), in
the launch configuration the benchmark times, with the ranged prefetch (scoring in several
launches) and with the fused one (one scoring launch with a host-gather wave per workgroup).
Every request is checked against the oracle (scores within 1e-4 T, the selection differing from
the oracle's only by tokens within that tolerance of its k-th score), and through properties
that hold at any size: the step's selection equals the exact top-k of its own scores, every
selected token is resident with its row equal to the host backup bit for bit, and the pool's
maps stay a bijection."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from dsa_indexer_top_amd.runner import DecodeRunner
from gpu_util import announce

pytestmark = pytest.mark.gpu
TOL = 1e-4


SMALL = gen.DecodeConfig("stress_small", 4, 6000, 256, "general", True, 0.5, 8, reserve=1024,
                         prefetch=True, seed=5)


@pytest.mark.parametrize("cfg", [SMALL, gen.CONFIGS["b64_128k"]], ids=["small", "full"])
def test_stress_step(cfg):
    announce("stress %s: drawing inputs" % cfg.name)
    inp = gen.make_decode_inputs(cfg)
    hb = B.HostBuffer(inp.n_host * 576 * 2)
    try:
        host_kv = hb.array.view(np.uint16).reshape(inp.n_host, 576)
        gen.fill_latent_rows(cfg.seed, host_kv)
        n_rows, max_len = len(inp.key_len), int(inp.key_len.max())
        dq, dw, dk = (torch.from_numpy(a).cuda() for a in (inp.q, inp.w, inp.k))
        dks = torch.from_numpy(inp.k_scale).cuda()
        dkb, dkl = torch.from_numpy(inp.key_begin).cuda(), torch.from_numpy(inp.key_len).cuda()
        sc = torch.empty((n_rows, max_len), dtype=torch.float32, device="cuda")
        sel = torch.empty((n_rows, cfg.topk), dtype=torch.int32, device="cuda")
        tws = torch.empty(B.topk_workspace_bytes(n_rows, max_len), dtype=torch.uint8, device="cuda")
        B.index_scores(dq, dw, dk, dks, dkb, dkl, max_len, sc)
        B.topk(sc, dkl, max_len, cfg.topk, sel, tws)
        want_idx = sel.cpu().numpy()
        del dq, dw, dk, dks, dkb, dkl, sc, sel, tws
        pool = gen.make_pool_state(inp, want_idx, host_kv)
        announce("stress %s: the oracle's scores of every request" % cfg.name)
        ref = []
        for r in range(n_rows):
            sl = slice(r, r + 1)
            args = (inp.q[sl], inp.w[sl], inp.k, inp.k_scale, inp.key_begin[sl], inp.key_len[sl])
            s = oracle.index_scores(*args)[0]
            ref.append((s, oracle.error_scale(*args)[0], oracle.topk_row(s, cfg.topk)))
        for mode in ("ranged", "fused"):
            announce("stress %s: captured step with %s prefetch" % (cfg.name, mode))
            rn = DecodeRunner(inp, pool, host_buf=hb, prefetch=mode)
            try:
                rn.capture()
                rn.replay()
                got = rn.results()
            finally:
                rn.close()
            _check_step(cfg, inp, host_kv, want_idx, got, mode, ref)
    finally:
        hb.close()


def _check_step(cfg, inp, host_kv, want_idx, got, mode, ref):
    n_rows = len(inp.key_len)
    assert got["status"] == 0, mode
    # the step's top-k is the exact top-k of the scores it computed
    assert np.array_equal(got["topk_idx"], want_idx), mode
    assert int(got["counters"][2]) > 0 and int(got["counters"][1]) >= int(got["counters"][2]), mode
    # every selected token resident, bit for bit; the maps a bijection
    idx = got["topk_idx"]
    rows, cols = np.nonzero(idx >= 0)
    assert len(rows) == n_rows * cfg.topk
    hosts = inp.req_to_host[inp.key_begin[rows] + idx[rows, cols]]
    st = oracle.PoolState(*(got["pool"][n] for n in ("free", "priority", "to_host",
                                                     "host_to_gpu", "indices_buf", "gpu_kv")))
    oracle.check_pool_invariants(st, host_kv, hosts, got["topk_slot"][rows, cols])
    # every request against the oracle: scores within 1e-4 T, and the selection differing from
    # the oracle's only by tokens within that tolerance of its k-th score
    for r in range(n_rows):
        s, T, want = ref[r]
        g = got["scores"][r, :len(s)].astype(np.float64)
        assert (np.abs(g - s) <= TOL * T).all(), "request %d scores (%s)" % (r, mode)
        kth = want[np.argmin(s[want])]
        for t in np.setxor1d(idx[r], want):
            assert abs(s[t] - s[kth]) <= TOL * (T[t] + T[kth]), "request %d token %d" % (r, t)
