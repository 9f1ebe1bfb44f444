"""Several layers in one decode step (ECHO page §5.1: the GPU pool is kept per layer, because
every layer selects its own tokens, while the host pool is kept per model, because it holds the
full backup whatever is evicted).  Each layer has its own indexer inputs and its own GPU pool;
all layers share one pinned host allocation laid out layer by layer; the layers' decode steps
are captured into one graph (echo_graph_begin / echo_graph_end) and replayed.  Each layer must
match the oracle's step on its own inputs and its own slice of the host pool, bit for bit (so no
layer touched another layer's pool or read another layer's rows).  Cases: three layers with
contiguous key caches, and the 61 layers of the pages' model with each layer's indexer-K cache in
64-token pages scattered in a random order, with the metadata footprint of every layer's pool
(4 N_H + 13 N_G bytes) checked against the arrays it is made of."""

import numpy as np
import pytest
import torch

import oracle
from dsa_indexer_top_amd import binding as B, inputs as gen
from gpu_util import announce, dev, host, assert_pool_equal

pytestmark = pytest.mark.gpu


def _run_layers(n_layers, lens, k, page_size=None, replays=1):
    layers = []
    for ell in range(n_layers):
        cfg = gen.DecodeConfig("L%d" % ell, len(lens), 0, k, "int", False, 0.6, 4, seed=90 + ell)
        layers.append(gen.make_decode_inputs(cfg, lengths=lens))
    n_host, n_rows = layers[0].n_host, len(lens)
    # the same tokens in every layer (one request's token s has one host row h for all layers)
    for inp in layers[1:]:
        inp.req_to_host[:] = layers[0].req_to_host
    row_bytes = 576 * 2
    hb = B.HostBuffer(n_layers * n_host * row_bytes)
    host_all = hb.array.view(np.uint16).reshape(n_layers, n_host, 576)
    for ell in range(n_layers):
        gen.fill_latent_rows(200 + ell, host_all[ell])
    want, runs = [], []
    try:
        for ell, inp in enumerate(layers):
            scores = oracle.index_scores(inp.q, inp.w, inp.k, None, inp.key_begin, inp.key_len)
            idx = oracle.topk_rows(scores, k)
            pool = gen.make_pool_state(inp, idx, host_all[ell])
            st0 = oracle.PoolState(pool.free.copy(), pool.priority.copy(), pool.to_host.copy(),
                                   pool.host_to_gpu.copy(), pool.indices_buf.copy(), pool.gpu_kv.copy())
            ws_, res = oracle.pool_step(st0, host_all[ell].copy(), idx, inp.key_begin,
                                        inp.req_to_host, pool.step_id)
            want.append((idx, ws_, res))
            d = dict(q=dev(inp.q), w=dev(inp.w), key_begin=dev(inp.key_begin),
                     key_len=dev(inp.key_len), req_to_host=dev(inp.req_to_host))
            if page_size:
                pk = gen.page_key_cache(inp.k, None, inp.key_begin, inp.key_len, page_size, seed=ell)
                d["k"], d["table"] = dev(pk.k_pages), dev(pk.page_table)
            else:
                d["k"] = dev(inp.k)
            live = {n: dev(getattr(pool, n)) for n in ("free", "priority", "to_host", "host_to_gpu",
                                                       "indices_buf", "gpu_kv")}
            meta = sum(live[n].numel() * live[n].element_size()
                       for n in ("free", "priority", "to_host", "host_to_gpu", "indices_buf"))
            assert meta == B.pool_metadata_bytes(n_host, inp.n_gpu) == oracle.metadata_bytes(n_host, inp.n_gpu)
            status = torch.zeros(1, dtype=torch.int32, device="cuda")
            P = B.make_pool(inp.n_gpu, n_host, live["free"], live["priority"], live["to_host"],
                            live["host_to_gpu"], live["indices_buf"], live["gpu_kv"],
                            hb.dev_ptr + ell * n_host * row_bytes, status)
            L = int(inp.key_len.max())
            out_t = dict(scores=torch.empty((n_rows, L), dtype=torch.float32, device="cuda"),
                         idx=torch.empty((n_rows, k), dtype=torch.int32, device="cuda"),
                         slot=torch.empty((n_rows, k), dtype=torch.int32, device="cuda"),
                         mh=torch.empty(n_rows * k, dtype=torch.int32, device="cuda"),
                         ms=torch.empty(n_rows * k, dtype=torch.int32, device="cuda"),
                         cnt=torch.zeros(8, dtype=torch.int32, device="cuda"))
            out = B.DecodeOut(*(out_t[n].data_ptr() for n in ("scores", "idx", "slot", "mh", "ms", "cnt")))
            args = B.DecodeArgs(d["q"].data_ptr(), d["w"].data_ptr(), d["k"].data_ptr(), None,
                                d["key_begin"].data_ptr(), d["key_len"].data_ptr(),
                                d["req_to_host"].data_ptr(), n_rows, L, k, pool.step_id, 0, 1, 4096,
                                95.0, 1, 1)
            if page_size:
                args.k_page_table = d["table"].data_ptr()
                args.k_page_size = page_size
                args.k_max_pages = d["table"].shape[1]
            ws = torch.empty(B.decode_workspace_bytes(args, inp.n_gpu), dtype=torch.uint8, device="cuda")
            runs.append(dict(d=d, live=live, status=status, P=P, out_t=out_t, out=out, args=args, ws=ws,
                             pool=pool))
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()

        def enqueue(st):
            for r in runs:
                B.decode_select(r["args"], r["P"], r["out"], r["ws"], st)

        g = B.CapturedGraph(enqueue, stream)
        try:
            for rep in range(replays):
                if rep:                                  # back to each layer's starting pool
                    for r in runs:
                        for n in r["live"]:
                            r["live"][n].copy_(torch.from_numpy(getattr(r["pool"], n)))
                        r["status"].zero_()
                    torch.cuda.synchronize()
                g.launch(stream)
                torch.cuda.synchronize()
                for ell, (r, (idx, want_state, res)) in enumerate(zip(runs, want)):
                    assert int(host(r["status"])[0]) == 0
                    assert np.array_equal(host(r["out_t"]["idx"]), idx), (rep, ell)
                    assert np.array_equal(host(r["out_t"]["slot"]), res.topk_slot), (rep, ell)
                    got = oracle.PoolState(*(host(r["live"][n]) for n in (
                        "free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv")))
                    assert_pool_equal(got, want_state, "replay %d layer %d" % (rep, ell))
                    # the recalled rows came from this layer's slice of the shared host pool
                    sel = res.miss_slot[:res.n_miss]
                    assert np.array_equal(got.gpu_kv[sel], host_all[ell][res.miss_host[:res.n_miss]])
                    assert res.n_miss > 0
        finally:
            g.close()
    finally:
        hb.close()


def test_layers_share_one_host_pool_in_one_graph():
    announce("three layers, one host pool, one graph")
    _run_layers(3, [3000, 1700], 128)


def test_61_layers_paged_keys_one_graph():
    announce("61 layers, paged indexer keys, one host pool, one graph")
    _run_layers(61, [4096, 2500], 256, page_size=64, replays=2)
