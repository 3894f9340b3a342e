"""CPU oracle for the W4A8 sparse-MoE decode layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU library never imports, links or calls it.  The arithmetic lives in
``moe_oracle.c`` (plain C, fp64 sums in natural order); this file only marshals numpy arrays.

Parity status of each function is recorded in ``PINS`` below and in the design notes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_SANITIZED_LIBS: a directory holding an AddressSanitizer / UndefinedBehaviorSanitizer build of
# the oracle (tests/sanitized.py) to load instead
LIB = os.path.join(os.environ.get("MOE_SANITIZED_LIBS") or _HERE, "libmoe_oracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-shared", "-fPIC", "-fopenmp"]

# Which independent check pins each oracle function (tests/test_oracle_*.py).
PINS = {
    "e2m1_decode": "OCP MX value table (16 codes)",
    "e8m0_decode": "closed form 2^(b-127), NaN at 255",
    "e4m3_decode": "generic minifloat enumeration; max 448, min subnormal 2^-9, NaN codes",
    "e4m3_encode": "exhaustive over all fp32 bit patterns vs nearest-of-256 by bisection, ties to even",
    "bf16_encode": "exhaustive over all fp32 bit patterns vs torch's round-to-nearest-even conversion",
    "route": "brute-force stable sort; softmax sums to 1; zero input gives ids 0..k-1",
    "moe_layer": "dense brute force over all experts; int64 exact block sums; metamorphic tests",
    "rmsnorm_bf16": "constant-vector closed form; power-of-two scale invariance",
    "residual_bf16": "bf16 round trip vs torch",
    "head": "argmax brute force; duplicate-row tie; BLAS GEMV special case",
    "mtp_accept": "hand cases: all, none, first-mismatch positions, a match after a mismatch is not accepted",
    "head_bf16": "BLAS GEMV special case; equals the FP8 head exactly on rows that are E4M3 values times a power of two",
    "route.bounds": "fp32 sums in natural, reversed, pairwise, permuted and the router kernel's order stay within it; "
                    "an adversarial half-ulp sum reaches at least half of it (a 16x looser bound is caught)",
    "head.bounds": "the same soundness and tightness checks for the FP8 and BF16 heads",
    "topk_margin_ok": "hand cases: a gap equal to the bound sum fails, a failing pair at rank 3 and at rank k fails",
    "argmax_margin_ok": "hand cases: a gap equal to the bound sum fails, a tie fails",
}


class _Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_shared", ctypes.c_int32), ("inter", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w13_s", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_s", ctypes.c_void_p)]


class _Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "bounds", "ids", "w", "sx", "qx", "g", "u", "h", "sh", "qh", "d")]


_lib = None


def build(force: bool = False) -> str:
    if os.environ.get("MOE_SANITIZED_LIBS"):
        return LIB  # built by tests/sanitized.py
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.check_call(["gcc", *GCC_FLAGS, SRC, "-o", LIB, "-lm"])
    return LIB


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.oracle_e2m1_decode.restype = ctypes.c_double
    L.oracle_e2m1_decode.argtypes = [ctypes.c_uint32]
    L.oracle_e8m0_decode.restype = ctypes.c_double
    L.oracle_e8m0_decode.argtypes = [ctypes.c_uint32]
    L.oracle_e4m3_decode.restype = ctypes.c_double
    L.oracle_e4m3_decode.argtypes = [ctypes.c_uint32]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    L.oracle_bf16_encode.restype = ctypes.c_uint16
    L.oracle_bf16_encode.argtypes = [ctypes.c_float]
    L.oracle_bf16_decode.restype = ctypes.c_float
    L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    for n in ("oracle_e4m3_encode_array", "oracle_bf16_encode_array"):
        getattr(L, n).restype = None
        getattr(L, n).argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
    L.oracle_set_threads.restype = None
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_max_threads.restype = ctypes.c_int
    L.oracle_max_threads.argtypes = []
    L.oracle_route.restype = ctypes.c_int
    L.oracle_route.argtypes = [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.oracle_moe_layer.restype = ctypes.c_int
    L.oracle_moe_layer.argtypes = [ctypes.POINTER(_Shape), ctypes.POINTER(_Weights), ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(_Trace)]
    L.oracle_rmsnorm_bf16.restype = None
    L.oracle_rmsnorm_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.oracle_residual_bf16.restype = None
    L.oracle_residual_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p]
    L.oracle_head_quantize.restype = None
    L.oracle_head_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    L.oracle_head_logits_bf16.restype = None
    L.oracle_head_logits_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.oracle_head_logits.restype = None
    L.oracle_head_logits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = _load(LIB)
    return _lib


class using:
    """Context manager that routes every oracle call to another build of ``moe_oracle.c``
    (the mutation tests compile deliberately broken copies of it)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    """Threads for the oracle's loops over independent output rows (1 = single-threaded, the
    default); results do not depend on it."""
    lib().oracle_set_threads(n)


def max_threads() -> int:
    return lib().oracle_max_threads()


# ---- codecs ------------------------------------------------------------------------------------

def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(code)


def e8m0_decode(b: int) -> float:
    return lib().oracle_e8m0_decode(b)


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(code)


def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(v), _p(out), v.size)
    return out


def bf16_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_encode_array(_p(v), _p(out), v.size)
    return out


def bf16_decode(b) -> np.ndarray:
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


# ---- MoE layer ---------------------------------------------------------------------------------

def _shape(s) -> _Shape:
    return _Shape(s.hidden, s.num_experts, s.top_k, s.num_shared, s.inter)


def route(shape, router, x) -> dict:
    """Routing of T tokens: logits/bounds [T][E] (fp64), ids [T][k], w [T][k] (fp64)."""
    router = _c(router, np.uint16)
    x = _c(x, np.uint16).reshape(-1, shape.hidden)
    T = x.shape[0]
    out = {"logits": np.empty((T, shape.num_experts)), "bounds": np.empty((T, shape.num_experts)),
           "ids": np.empty((T, shape.top_k), dtype=np.int32), "w": np.empty((T, shape.top_k))}
    sh = _shape(shape)
    rc = lib().oracle_route(ctypes.byref(sh), _p(router), _p(x), T, _p(out["logits"]), _p(out["bounds"]),
                            _p(out["ids"]), _p(out["w"]))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc})")
    return out


def moe_layer(shape, router, experts: dict, x, trace: bool = True):
    """One layer.  ``experts`` maps expert index (num_experts = shared) to the dict of canonical
    tensors ``w13, w13_s, w2, w2_s``; only selected experts need be present.
    Returns (y fp32 [T][H], trace dict or None)."""
    router = _c(router, np.uint16)
    x = _c(x, np.uint16).reshape(-1, shape.hidden)
    T = x.shape[0]
    n = shape.num_experts + shape.num_shared
    keep = []
    tabs = {}
    for name in ("w13", "w13_s", "w2", "w2_s"):
        arr = (ctypes.c_void_p * n)()
        for e, t in experts.items():
            a = _c(t[name], np.uint8)
            keep.append(a)
            arr[e] = a.ctypes.data
        tabs[name] = arr
    W = _Weights(_p(router), ctypes.cast(tabs["w13"], ctypes.c_void_p), ctypes.cast(tabs["w13_s"], ctypes.c_void_p),
                 ctypes.cast(tabs["w2"], ctypes.c_void_p), ctypes.cast(tabs["w2_s"], ctypes.c_void_p))
    y = np.empty((T, shape.hidden), dtype=np.float32)
    slots = shape.top_k + shape.num_shared
    I, H, E, k = shape.inter, shape.hidden, shape.num_experts, shape.top_k
    tr = None
    trp = None
    if trace:
        tr = {"logits": np.empty((T, E)), "bounds": np.empty((T, E)), "ids": np.empty((T, k), dtype=np.int32),
              "w": np.empty((T, k)), "sx": np.empty(T, dtype=np.float32), "qx": np.empty((T, H), dtype=np.uint8),
              "g": np.empty((T, slots, I)), "u": np.empty((T, slots, I)),
              "h": np.empty((T, slots, I), dtype=np.float32), "sh": np.empty((T, slots), dtype=np.float32),
              "qh": np.empty((T, slots, I), dtype=np.uint8), "d": np.empty((T, slots, H))}
        trp = _Trace(*[_p(tr[f]) for f, _ in _Trace._fields_])
    sh = _shape(shape)
    rc = lib().oracle_moe_layer(ctypes.byref(sh), ctypes.byref(W), _p(x), T, _p(y),
                                ctypes.byref(trp) if trp is not None else None)
    if rc != 0:
        raise ValueError(f"oracle_moe_layer failed ({rc})")
    return y, tr


def rmsnorm_bf16(x) -> np.ndarray:
    x = _c(x, np.uint16)
    T, H = x.shape
    out = np.empty_like(x)
    lib().oracle_rmsnorm_bf16(_p(x), T, H, _p(out))
    return out


def residual_bf16(x, y) -> np.ndarray:
    x = _c(x, np.uint16)
    y = _c(y, np.float32)
    T, H = x.shape
    out = np.empty_like(x)
    lib().oracle_residual_bf16(_p(x), _p(y), T, H, _p(out))
    return out


# ---- LM head -----------------------------------------------------------------------------------

def head_quantize(W):
    W = _c(W, np.float32)
    V, H = W.shape
    Wq = np.empty((V, H), dtype=np.uint8)
    s = np.empty(V, dtype=np.float32)
    lib().oracle_head_quantize(_p(W), V, H, _p(Wq), _p(s))
    return Wq, s


def head_logits(Wq, scale, x, want_logits: bool = True, want_bounds: bool = True):
    Wq = _c(Wq, np.uint8)
    scale = _c(scale, np.float32)
    x = _c(x, np.uint16)
    V, H = Wq.shape
    T = x.shape[0]
    lg = np.empty((T, V)) if want_logits else None
    bd = np.empty((T, V)) if want_bounds else None
    am = np.empty(T, dtype=np.int32)
    lib().oracle_head_logits(_p(Wq), _p(scale), V, H, _p(x), T, _p(lg), _p(bd), _p(am))
    return lg, bd, am


def head_logits_bf16(W, x, want_logits: bool = True, want_bounds: bool = True):
    """The unquantised BF16 head (W bf16 bits [V][H]): fp64 logits, fp32 error bounds, argmax."""
    W = _c(W, np.uint16)
    x = _c(x, np.uint16)
    V, H = W.shape
    T = x.shape[0]
    lg = np.empty((T, V)) if want_logits else None
    bd = np.empty((T, V)) if want_bounds else None
    am = np.empty(T, dtype=np.int32)
    lib().oracle_head_logits_bf16(_p(W), V, H, _p(x), T, _p(lg), _p(bd), _p(am))
    return lg, bd, am


def mtp_accept(argmax, draft) -> int:
    """Greedy acceptance of a speculative verify step: position i's target token argmax[i] is the
    model's next token after position i, and draft[i] the drafted token for position i + 1.  The
    drafts are accepted while they equal the target's tokens; returns how many were accepted
    (0 .. len(draft)); the step then emits those drafts plus argmax[accepted]."""
    n = 0
    while n < len(draft) and int(argmax[n]) == int(draft[n]):
        n += 1
    return n


# ---- margins (well-posedness of integer results under fp32 evaluation) -----------------------

def topk_margin_ok(logits, bounds, k: int) -> bool:
    """True when the first k+1 logits in (value desc, index asc) order are separated by more
    than the sum of their fp32 error bounds, so the ordered ids cannot change under any fp32
    summation order."""
    order = np.lexsort((np.arange(logits.size), -logits))[: k + 1]
    for a, b in zip(order[:-1], order[1:]):
        if logits[a] - logits[b] <= bounds[a] + bounds[b]:
            return False
    return True


def argmax_margin_ok(logits, bounds) -> bool:
    order = np.lexsort((np.arange(logits.size), -logits))[:2]
    a, b = order
    return logits[a] - logits[b] > bounds[a] + bounds[b]
