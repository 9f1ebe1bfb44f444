"""pytest plugin that runs the GPU parity tests against the host build of the library.

Loaded with `-p emu_plugin` (this directory on PYTHONPATH) in a process started with clang's
AddressSanitizer runtime preloaded and ECHO_EMU_LIB naming the library build_emu.py wrote.
torch tensors asked for on "cuda" are made on the CPU, so the library receives host pointers;
uninitialised allocations (torch.empty, empty_like) are filled with a 0xBE byte pattern so that
a kernel that reads memory it never wrote sees garbage, as it would on the GPU.  Streams are
stand-ins with distinct non-null handles.  Test infrastructure only.
"""
import contextlib
import os

import torch

POISON = 0xBE


class _Stream:
    _next = 0x1000

    def __init__(self, *a, **k):
        _Stream._next += 0x10
        self.cuda_stream = _Stream._next

    def wait_stream(self, *a, **k):
        pass

    def synchronize(self):
        pass


_CURRENT = _Stream()


def _is_cuda(d):
    if isinstance(d, torch.device):
        return d.type == "cuda"
    return isinstance(d, str) and d.startswith("cuda")


def _on_cpu(fn, poison=False):
    def f(*a, **kw):
        if _is_cuda(kw.get("device")):
            kw["device"] = "cpu"
        t = fn(*a, **kw)
        if poison and t.numel() and t.is_contiguous():
            t.view(torch.uint8).fill_(POISON)
        return t
    return f


def _install():
    for name in ("full", "zeros", "ones", "randn", "rand", "randint", "arange", "tensor",
                 "as_tensor", "zeros_like", "full_like", "ones_like", "linspace"):
        setattr(torch, name, _on_cpu(getattr(torch, name)))
    for name in ("empty", "empty_like"):
        setattr(torch, name, _on_cpu(getattr(torch, name), poison=True))
    torch.cuda.is_available = lambda: True
    torch.cuda.synchronize = lambda *a, **k: None
    torch.cuda.set_device = lambda *a, **k: None
    torch.cuda.Stream = _Stream
    torch.cuda.current_stream = lambda *a, **k: _CURRENT
    torch.cuda.stream = lambda s: contextlib.nullcontext()
    to = torch.Tensor.to

    def to_cpu(self, *a, **kw):
        a = tuple("cpu" if _is_cuda(x) else x for x in a)
        if _is_cuda(kw.get("device")):
            kw["device"] = "cpu"
        return to(self, *a, **kw)
    torch.Tensor.to = to_cpu
    torch.Tensor.cuda = lambda self, *a, **k: self.clone()
    from dsa_indexer_top_amd import binding
    binding.LIB_PATH = os.environ["ECHO_EMU_LIB"]


def pytest_configure(config):
    _install()
