"""Builds a host (CPU) version of libecho.so from the HIP sources, for AddressSanitizer runs.

The sources are copied and rewritten mechanically: <hip/hip_runtime.h> becomes hip_cpu.h, the
amdgcn builtins become the functions of emu_runtime.cpp, `kernel<<<grid, block, lds, stream>>>(
args)` becomes `emu::launch_kernel(dim3(grid), dim3(block), &kernel, args)`, and every
__shared__ object is registered for poisoning.  clang compiles the result as C++17 with
-fsanitize=address into one shared library that exports the same C ABI as the GPU build.

    python tests/emu/build_emu.py [--thread] [CSRC_DIR INCLUDE_DIR OUT_DIR]

Test infrastructure only: nothing in the package loads this library.
"""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CLANG = os.environ.get("ECHO_EMU_CXX", "/opt/rocm/llvm/bin/clang++")
DEFAULT_OUT = os.path.join(ROOT, "_build", "emu")
LIB_NAME = "libecho_emu.so"


def sanitizer_runtime(name="asan"):
    """Path of clang's shared sanitizer runtime ("asan" or "tsan"), or None."""
    try:
        d = subprocess.run([CLANG, "-print-resource-dir"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    p = os.path.join(d, "lib", "linux", "libclang_rt.%s-x86_64.so" % name)
    return p if os.path.exists(p) else None


def asan_runtime():
    return sanitizer_runtime("asan")


def _match(s, i, open_c, close_c):
    d = 0
    for j in range(i, len(s)):
        if s[j] == open_c:
            d += 1
        elif s[j] == close_c:
            d -= 1
            if d == 0:
                return j
    raise ValueError("unbalanced %s at %d" % (open_c, i))


def _split_top(s):
    out, d, cur = [], 0, ""
    for ch in s:
        d += ch in "([{"
        d -= ch in ")]}"
        if ch == "," and d == 0:
            out.append(cur)
            cur = ""
        else:
            cur += ch
    out.append(cur)
    return out


def _name_start(s, end):
    """Start of the `name<template args>` expression that ends at `end`."""
    j = end
    while j > 0 and s[j - 1] in " \t":
        j -= 1
    if s[j - 1] == ">":
        d, k = 0, j - 1
        while True:
            d += s[k] == ">"
            d -= s[k] == "<"
            if d == 0:
                break
            k -= 1
        j = k
    while j > 0 and (s[j - 1].isalnum() or s[j - 1] in "_:"):
        j -= 1
    return j


SHARED = re.compile(r"__shared__\s+([^;]*?)\b([A-Za-z_]\w*)\s*((?:\[[^\]]*\])*)\s*;")
# An empty asm statement with register operands only pins the order of GPU instructions; the
# CPU build drops it (x86 has no register class for an 8 x 32-bit operand).
PIN = re.compile(r'asm\s+volatile\s*\(\s*""\s*:[^;]*\)\s*;')


def transform(src):
    src = src.replace("#include <hip/hip_runtime.h>", '#include "hip_cpu.h"')
    src = src.replace("__builtin_amdgcn_", "emu_amdgcn_")
    src = src.replace("__builtin_nontemporal_load", "emu_nontemporal_load")
    src = PIN.sub("((void)0);", src)
    src = SHARED.sub(lambda m: "static %s%s%s; static const bool %s_emu_lds = "
                     "(emu::lds_register(&%s, sizeof(%s)), true);" % (
                         m.group(1), m.group(2), m.group(3), m.group(2), m.group(2), m.group(2)),
                     src)
    out, pos = [], 0
    while True:
        i = src.find("<<<", pos)
        if i < 0:
            out.append(src[pos:])
            break
        st = _name_start(src, i)
        name = src[st:i].strip()
        e = src.find(">>>", i)
        cfg = _split_top(src[i + 3:e])
        k = e + 3
        while src[k] in " \t\\\n":
            k += 1
        a_end = _match(src, k, "(", ")")
        args = src[k + 1:a_end]
        call = "emu::launch_kernel(dim3(%s), dim3(%s), &%s" % (cfg[0].strip(), cfg[1].strip(), name)
        if args.strip():
            call += ", " + args
        out += [src[pos:st], call + ")"]
        pos = a_end + 1
    return "".join(out)


def build(csrc=None, include=None, out=DEFAULT_OUT, sanitizer="address"):
    """sanitizer: "address" (every source) or "thread" (the library's sources; the fiber
    runtime itself stays uninstrumented and reports the fibers to ThreadSanitizer)."""
    csrc = os.path.abspath(csrc or os.path.join(ROOT, "dsa_indexer_top_amd", "csrc"))
    include = os.path.abspath(include or os.path.join(ROOT, "include"))
    out = os.path.abspath(out)
    shutil.rmtree(out, ignore_errors=True)
    cdir = os.path.join(out, "src", "csrc")          # the sources include "../../include/echo.h"
    os.makedirs(cdir)
    os.symlink(include, os.path.join(out, "include"))
    shutil.copy(os.path.join(HERE, "hip_cpu.h"), cdir)
    units = []
    for f in sorted(os.listdir(csrc)):
        p = os.path.join(csrc, f)
        if not os.path.isfile(p):
            continue
        with open(p) as fh:
            s = transform(fh.read())
        with open(os.path.join(cdir, f), "w") as fh:
            fh.write(s)
        if f.endswith((".hip", ".cpp")):
            units.append(os.path.join(cdir, f))
    runtime = os.path.join(HERE, "emu_runtime.cpp")
    units.append(runtime)
    flags = ["-std=c++17", "-g", "-O1", "-fPIC", "-fno-omit-frame-pointer", "-Wno-unused-variable",
             "-I", cdir]
    if sanitizer == "address":
        # the kernels also under the alignment check: a vector access at an address that is not
        # a multiple of its size faults on the GPU
        kflags = ["-fsanitize=address,alignment", "-fno-sanitize-recover=alignment"]
        rflags = ["-fsanitize=address", "-DEMU_ASAN"]
    elif sanitizer == "thread":
        kflags, rflags = ["-fsanitize=thread"], ["-DEMU_TSAN"]
    else:
        raise ValueError(sanitizer)

    def compile_one(u):
        o = os.path.join(out, os.path.basename(u) + ".o")
        extra = rflags if u == runtime else kflags
        r = subprocess.run([CLANG, "-x", "c++", *flags, *extra, "-c", u, "-o", o], capture_output=True,
                           text=True)
        if r.returncode:
            raise RuntimeError("emulation build failed for %s:\n%s" % (u, r.stderr[-6000:]))
        return o

    with cf.ThreadPoolExecutor(max_workers=min(8, len(units))) as ex:
        objs = list(ex.map(compile_one, units))
    lib = os.path.join(out, LIB_NAME)
    link_san = "address,alignment" if sanitizer == "address" else sanitizer
    r = subprocess.run([CLANG, "-shared", "-fsanitize=" + link_san, "-shared-libsan", "-o", lib, *objs],
                       capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("emulation link failed:\n%s" % r.stderr[-4000:])
    return lib


if __name__ == "__main__":
    a = sys.argv[1:]
    san = "address"
    if a and a[0] in ("--thread", "--address"):
        san, a = a[0][2:], a[1:]
    print(build(*a, sanitizer=san))
