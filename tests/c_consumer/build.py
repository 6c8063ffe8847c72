"""Compile the plain-C consumer of the C ABI (``moe_layer.c``) with gcc,
against ``include/`` and the built library. Run by ``__graft_entry__.build()``
after the library, so the binary is in the tree before any GPU run; the test
compiles it itself when it is missing or older than its source."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "moe_layer.c")
EXE = os.path.join(HERE, "moe_layer")
PKG = os.path.join(ROOT, "token_dispatch_grouped_amd")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ROCM = "/opt/rocm"


def command(out: str) -> list:
    gcc = shutil.which("gcc") or "gcc"
    return [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), SRC,
            "-L", PKG, "-lmoe_mi355x", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out]


def build(out: str = EXE) -> str:
    """Compile the consumer to ``out``; raises with the compiler's output on failure."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} not found: build the HIP library first")
    cmd = command(out)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def current() -> str:
    """The in-tree binary, rebuilt first if it is missing or older than its source or the library."""
    if (not os.path.exists(EXE) or os.path.getmtime(EXE) < os.path.getmtime(SRC)
            or os.path.getmtime(EXE) < os.path.getmtime(LIB)):
        build(EXE)
    return EXE
