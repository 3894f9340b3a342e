"""Compiles the C-ABI library libmoe_decode.so (HIP, gfx950) in-tree."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libmoe_decode.so")
SOURCES = [os.path.join(_HERE, "csrc", f) for f in ("moe_kernels.hip", "moe_api.cpp", "head_kernels.hip", "head_api.cpp")]


def build(hipcc: str, flags: list) -> str:
    """Compiles every source into LIB with the given hipcc flags (which carry -shared -fPIC)."""
    tmp = LIB + ".tmp"
    subprocess.check_call([hipcc, *flags, *SOURCES, "-o", tmp], cwd=_HERE)
    os.replace(tmp, LIB)
    return LIB
