"""Helpers for GPU tests: move seeded numpy inputs to the device, print the case first."""

import sys

import numpy as np


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def decode_inputs_to_dev(inp):
    d = dict(q=dev(inp.q), w=dev(inp.w), k=dev(inp.k),
             k_scale=None if inp.k_scale is None else dev(inp.k_scale),
             key_begin=dev(inp.key_begin), key_len=dev(inp.key_len),
             req_to_host=dev(inp.req_to_host))
    return d


class DevPool:
    """Device copy of a pool state + pinned mapped host backup, with the ctypes struct."""

    def __init__(self, free, priority, to_host, host_to_gpu, indices_buf, gpu_kv, host_kv,
                 coherent=False):
        import torch
        from dsa_indexer_top_amd import binding as B
        self.free = dev(free)
        self.priority = dev(priority)
        self.to_host = dev(to_host)
        self.host_to_gpu = dev(host_to_gpu)
        self.indices_buf = dev(indices_buf)
        self.gpu_kv = dev(gpu_kv)
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.hostbuf = B.HostBuffer(host_kv.nbytes, coherent=coherent)
        self.host_kv = self.hostbuf.array.view(np.uint16).reshape(host_kv.shape)
        self.host_kv[...] = host_kv
        self.n_gpu, self.n_host = len(free), len(host_to_gpu)
        self.pool = B.make_pool(self.n_gpu, self.n_host, self.free, self.priority, self.to_host,
                                self.host_to_gpu, self.indices_buf, self.gpu_kv,
                                self.hostbuf.dev_ptr, self.status)

    def state(self):
        import oracle
        return oracle.PoolState(host(self.free), host(self.priority), host(self.to_host),
                                host(self.host_to_gpu), host(self.indices_buf), host(self.gpu_kv))

    def close(self):
        self.hostbuf.close()


def assert_pool_equal(got, want, what=""):
    for name in ("free", "priority", "to_host", "host_to_gpu", "indices_buf", "gpu_kv"):
        a, b = getattr(got, name), getattr(want, name)
        if not np.array_equal(a, b):
            bad = np.flatnonzero((a != b).reshape(len(a), -1).any(axis=1))
            raise AssertionError("%s %s differs at %d entries, first %d: gpu %r oracle %r" % (
                what, name, len(bad), bad[0], a[bad[0]], b[bad[0]]))
