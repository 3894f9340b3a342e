"""Seeded synthetic inputs for the MXFP4 sparse-MoE decode layer.

Thin ctypes wrapper over ``synth_host.c`` (host generator) and ``synth_device.hip`` (its
integer-only device twin).  The generator's definition is in the header of ``synth_host.c``.
This module draws random numbers and lays them out; it contains none of the MoE method's
arithmetic, so the oracle and the GPU library can both consume its bytes without sharing code.

Distributions (one MoE layer): router rows ~ N(0, 0.02) rounded to bf16; activations
~ N(0, 1) rounded to bf16; E2M1 codes uniform over all 16 codes; E8M0 block scales uniform over
exponents -6..-2; LM-head weights ~ N(0, 0.02) in fp32.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZED_LIBS: a directory holding an AddressSanitizer / UndefinedBehaviorSanitizer build of
# the host generator (tests/sanitized.py) to load instead
HOST_LIB = os.path.join(os.environ.get("MOE_SANITIZED_LIBS") or _HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(_HERE, "libsynth_device.so")

TENSOR_ROUTER, TENSOR_W13, TENSOR_W13S, TENSOR_W2, TENSOR_W2S, TENSOR_X, TENSOR_HEAD = range(7)

ROUTER_SIGMA = 0.02
X_SIGMA = 1.0
HEAD_SIGMA = 0.02

_host = None
_dev = None


def _u64(v):
    return ctypes.c_uint64(v & 0xFFFFFFFFFFFFFFFF)


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.c_uint32]
        lib.synth_hash.restype = ctypes.c_uint64
        lib.synth_hash.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        for name in ("synth_codes", "synth_scales"):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double]
        _host = lib
    return _host


def device_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEVICE_LIB):
            raise RuntimeError(f"{DEVICE_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEVICE_LIB)
        for name in ("synth_dev_codes", "synth_dev_scales"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                           ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        _dev = lib
    return _dev


def key(seed: int, layer: int, tensor: int, expert: int, attempt: int) -> int:
    return host_lib().synth_key(_u64(seed), layer, tensor, expert, attempt)


def codes(n: int, k: int, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    host_lib().synth_codes(out.ctypes.data, i0, n, _u64(k))
    return out


def scales(n: int, k: int, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    host_lib().synth_scales(out.ctypes.data, i0, n, _u64(k))
    return out


def normal_bf16(n: int, k: int, sigma: float, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().synth_normal_bf16(out.ctypes.data, i0, n, _u64(k), sigma)
    return out


def normal_f32(n: int, k: int, sigma: float, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().synth_normal_f32(out.ctypes.data, i0, n, _u64(k), sigma)
    return out


@dataclass(frozen=True)
class Shape:
    hidden: int
    num_experts: int
    top_k: int
    num_shared: int
    inter: int

    @property
    def w13_bytes(self):  # E2M1 codes of one expert's gate+up rows, [2I][H/2]
        return 2 * self.inter * self.hidden // 2

    @property
    def w13s_bytes(self):  # E8M0 scales, [2I][H/32]
        return 2 * self.inter * self.hidden // 32

    @property
    def w2_bytes(self):  # [H][I/2]
        return self.hidden * self.inter // 2

    @property
    def w2s_bytes(self):  # [H][I/32]
        return self.hidden * self.inter // 32


TINY = Shape(hidden=256, num_experts=16, top_k=2, num_shared=1, inter=64)
FLASH = Shape(hidden=2560, num_experts=512, top_k=8, num_shared=1, inter=768)
HEAD_VOCAB = 157184


def router(shape: Shape, seed: int, layer: int = 0, attempt: int = 0) -> np.ndarray:
    """bf16 bits [E][H]."""
    k = key(seed, layer, TENSOR_ROUTER, 0, attempt)
    return normal_bf16(shape.num_experts * shape.hidden, k, ROUTER_SIGMA).reshape(shape.num_experts, shape.hidden)


def tokens(hidden: int, seed: int, T: int, attempt: int = 0, layer: int = 0) -> np.ndarray:
    """bf16 bits [T][H]; token t is drawn with the expert coordinate set to t."""
    out = np.empty((T, hidden), dtype=np.uint16)
    for t in range(T):
        out[t] = normal_bf16(hidden, key(seed, layer, TENSOR_X, t, attempt), X_SIGMA)
    return out


def tokens_correlated(hidden: int, seed: int, T: int, rho: float, attempt: int = 0, layer: int = 0) -> np.ndarray:
    """bf16 bits [T][H] of T tokens with a common component: token 0 is z_0 and token t >= 1 is
    rho z_0 + sqrt(1 - rho^2) z_t, with z_t ~ N(0, 1) in fp32 drawn as in tokens() and the mix
    rounded once to bf16 (nearest, ties to even).  Their router scores are correlated, so their
    top-k sets overlap, as for the positions of one speculative verify step."""
    z = [normal_f32(hidden, key(seed, layer, TENSOR_X, t, attempt), X_SIGMA).astype(np.float64) for t in range(T)]
    mix = np.empty((T, hidden), dtype=np.float32)
    mix[0] = z[0]
    for t in range(1, T):
        mix[t] = rho * z[0] + np.sqrt(1.0 - rho * rho) * z[t]
    u = mix.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def tokens_wide_range(hidden: int, seed: int, T: int, attempt: int = 0) -> np.ndarray:
    """bf16 bits [T][H] with a wide dynamic range inside every block of 32: one element of magnitude
    4 (random position and sign) and 31 of magnitude in [0.12, 0.24] / 112 (random sign), so that
    after per-token E4M3 quantisation (amax 4 -> 448, scale 1/112) every block holds one code of 448
    and 31 codes between 2^-3 and 2^-2.  Random bytes come from the E2M1-code stream with the expert
    coordinate 64 + t; magnitudes are rounded once to bf16 (nearest, ties to even)."""
    out = np.empty((T, hidden), dtype=np.float32)
    for t in range(T):
        r = codes(2 * hidden, key(seed, 0, TENSOR_X, 64 + t, attempt)).astype(np.int64)
        mag = (0.12 + 0.12 * r[:hidden] / 255.0) / 112.0
        for b in range(hidden // 32):
            mag[32 * b + (r[hidden + 32 * b] & 31)] = 4.0
        sign = np.where(r[hidden:] & 1, -1.0, 1.0)
        out[t] = (sign * mag).astype(np.float32)
    u = out.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def expert(shape: Shape, seed: int, layer: int, e: int) -> dict:
    """Canonical MXFP4 tensors of expert e (index num_experts is the shared expert).

    w13   [2I][H/2]  E2M1 codes, rows 0..I-1 gate, I..2I-1 up, low nibble = even k
    w13_s [2I][H/32] E8M0 scales, one per 32 consecutive k
    w2    [H][I/2]   E2M1 codes of the down projection
    w2_s  [H][I/32]  E8M0 scales
    """
    H, I = shape.hidden, shape.inter
    return {
        "w13": codes(shape.w13_bytes, key(seed, layer, TENSOR_W13, e, 0)).reshape(2 * I, H // 2),
        "w13_s": scales(shape.w13s_bytes, key(seed, layer, TENSOR_W13S, e, 0)).reshape(2 * I, H // 32),
        "w2": codes(shape.w2_bytes, key(seed, layer, TENSOR_W2, e, 0)).reshape(H, I // 2),
        "w2_s": scales(shape.w2s_bytes, key(seed, layer, TENSOR_W2S, e, 0)).reshape(H, I // 32),
    }


def head_weights(vocab: int, hidden: int, seed: int, row0: int = 0, rows: int | None = None) -> np.ndarray:
    """fp32 [rows][H] slice of the LM-head matrix ~ N(0, 0.02)."""
    rows = vocab - row0 if rows is None else rows
    k = key(seed, 0, TENSOR_HEAD, 0, 0)
    return normal_f32(rows * hidden, k, HEAD_SIGMA, i0=row0 * hidden).reshape(rows, hidden)


def _stream_ptr(stream):
    if stream is None:
        return None
    return ctypes.c_void_p(int(stream))


def fill_experts_device(w13, w13_s, w2, w2_s, shape: Shape, seed: int, layer: int, expert0: int = 0,
                        stream=None) -> None:
    """Fill device tensors [n][...] (uint8, contiguous) for experts expert0 .. expert0+n-1 in place.

    The tensors are any objects with ``data_ptr()`` and ``shape[0]`` (torch tensors on the GPU).
    """
    lib = device_lib()
    n = w13.shape[0]
    sp = _stream_ptr(stream)
    for t, tid, per in ((w13, TENSOR_W13, shape.w13_bytes), (w2, TENSOR_W2, shape.w2_bytes)):
        rc = lib.synth_dev_codes(ctypes.c_void_p(t.data_ptr()), per, n, expert0, _u64(seed), layer, tid, 0, sp)
        if rc != 0:
            raise RuntimeError(f"synth_dev_codes failed with {rc}")
    for t, tid, per in ((w13_s, TENSOR_W13S, shape.w13s_bytes), (w2_s, TENSOR_W2S, shape.w2s_bytes)):
        rc = lib.synth_dev_scales(ctypes.c_void_p(t.data_ptr()), per, n, expert0, _u64(seed), layer, tid, 0, sp)
        if rc != 0:
            raise RuntimeError(f"synth_dev_scales failed with {rc}")
