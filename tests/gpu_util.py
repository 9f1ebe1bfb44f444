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
