"""Python binding of the MI355X W4A8 sparse-MoE decode library (``libmoe_decode.so``).

Argument marshalling only: every step of the decode path runs in the library's HIP kernels.  The
functions keep the C names (``include/moe_decode.h`` documents each one).  Tensors are torch
tensors on the GPU; only their ``data_ptr()`` crosses the boundary, together with the hipStream_t
of a torch stream (the current stream by default).  A missing library is an error, never a
fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_SANITIZED_LIBS: a directory holding an AddressSanitizer / UndefinedBehaviorSanitizer build of
# the library (host code instrumented; built by tests/sanitized.py) to load instead
LIB = os.path.join(os.environ.get("MOE_SANITIZED_LIBS") or _HERE, "libmoe_decode.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_DTYPE",
          -4: "MOE_ERR_OOM", -5: "MOE_ERR_HIP", -6: "MOE_ERR_NO_DEVICE", -7: "MOE_ERR_STATE"}
DT_BF16, DT_FP32, DT_E4M3, DT_E2M1X2, DT_E8M0 = 1, 2, 3, 4, 5
F_RMSNORM_INPUT = 0x1
F_DIRECT_LAUNCH = 0x2
F_JIT = 0x8
F_MFMA = 0x10
F_GENERIC = 0x20  # shape-generic kernels even for the flash layer shape

# every symbol the header declares
EXPORTS = ("moe_decode_create", "moe_decode_set_layer", "moe_decode_run", "moe_decode_query",
           "moe_decode_destroy", "moe_decode_check", "moe_decode_timing_enable", "moe_decode_timing_read", "fp8_head_create", "fp8_head_run", "fp8_head_destroy", "fp8_head_quantize", "bf16_head_create", "fp8_head_verify",
           "fp8_head_run_noalloc", "moe_probe_stream_read", "moe_status_string", "moe_last_error")
NOALLOC_MAX_VOCAB = 262144


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_shared", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("num_layers", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("router", Tensor), ("w13", Tensor), ("w13_s", Tensor), ("w2", Tensor), ("w2_s", Tensor)]


class Outputs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("x_out", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("x_trace", ctypes.c_void_p),
                ("x_scale", ctypes.c_void_p), ("x_codes", ctypes.c_void_p)]


class Info(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("variant", ctypes.c_char * 64),
                ("weight_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                ("bytes_per_layer_t1", ctypes.c_uint64), ("layers_set", ctypes.c_int32),
                ("jit_from_cache", ctypes.c_int32), ("jit_compile_ms", ctypes.c_double),
                ("jit_code_object", ctypes.c_char * 512)]


# kernel classes of the timing record
TIMING_CLASSES = ("input", "router", "gateup", "requant", "down")


class Timing(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("runs", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("launches", ctypes.c_uint64 * 5), ("total_ms", ctypes.c_double * 5),
                ("gap_launches", ctypes.c_uint64 * 5), ("gap_ms", ctypes.c_double * 5)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        sig = {
            "moe_decode_create": [ctypes.POINTER(Config), vp, ctypes.POINTER(vp)],
            "moe_decode_set_layer": [vp, i32, ctypes.POINTER(LayerDesc), vp],
            "moe_decode_run": [vp, vp, i32, ctypes.POINTER(Outputs), vp],
            "moe_decode_query": [vp, ctypes.POINTER(Info)],
            "moe_decode_destroy": [vp],
            "moe_decode_check": [vp],
            "moe_decode_timing_enable": [vp, i32, i32],
            "moe_decode_timing_read": [vp, ctypes.POINTER(Timing)],
            "fp8_head_create": [i32, i32, Tensor, Tensor, vp, ctypes.POINTER(vp)],
            "fp8_head_run": [vp, vp, i32, vp, vp, vp],
            "fp8_head_destroy": [vp],
            "fp8_head_quantize": [i32, i32, Tensor, vp, vp, vp],
            "bf16_head_create": [i32, i32, Tensor, vp, ctypes.POINTER(vp)],
            "fp8_head_verify": [vp, vp, i32, vp, vp, vp, vp],
            "fp8_head_run_noalloc": [i32, i32, Tensor, Tensor, vp, i32, vp, vp, vp],
            "moe_probe_stream_read": [vp, ctypes.c_uint64, vp, i32, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _dtype_tag(t, byte_tag: int) -> int:
    """The tag of a torch tensor, from its own dtype: bfloat16 -> BF16, float32 -> FP32,
    float8_e4m3fn -> E4M3, float8_e8m0fnu -> E8M0, float4_e2m1fn_x2 -> E2M1X2; raw bytes (uint8)
    take the byte format of the slot they are passed in (E2M1X2, E8M0 or E4M3).  Any other dtype
    gets tag -1, which every slot rejects."""
    import torch
    fixed = {torch.bfloat16: DT_BF16, torch.float32: DT_FP32}
    for name, tag in (("float8_e4m3fn", DT_E4M3), ("float8_e8m0fnu", DT_E8M0), ("float4_e2m1fn_x2", DT_E2M1X2)):
        if hasattr(torch, name):
            fixed[getattr(torch, name)] = tag
    if t.dtype == torch.uint8:
        return byte_tag
    return fixed.get(t.dtype, -1)


def _check_buffer(t, name: str, nbytes: int) -> None:
    """t must be a contiguous tensor on the GPU holding exactly nbytes."""
    if not t.is_cuda:
        raise ValueError(f"{name}: not a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    got = t.numel() * t.element_size()
    if got != nbytes:
        raise ValueError(f"{name}: {got} bytes, expected {nbytes} ({tuple(t.shape)} {t.dtype})")


def _tensor(t, byte_tag: int, name: str = "tensor", nbytes: int | None = None) -> Tensor:
    """A torch tensor, tagged from its own dtype (see _dtype_tag), or a (tensor, tag) pair with an
    explicit tag.  With nbytes, the tensor's placement, layout and size are checked first."""
    if isinstance(t, tuple):
        t, tag = t
    else:
        tag = None if t is None else _dtype_tag(t, byte_tag)
    if t is not None and nbytes is not None:
        _check_buffer(t, name, nbytes)
    return Tensor(None if t is None else t.data_ptr(), -1 if tag is None else tag)


class Handle(ctypes.c_void_p):
    """Opaque handle of the library, with the sizes it was created for (used by the argument
    checks of this binding)."""


def moe_decode_create(hidden: int, num_experts: int, top_k: int, num_shared: int, inter: int, max_tokens: int,
                      num_layers: int = 1, flags: int = 0, stream=None) -> ctypes.c_void_p:
    cfg = Config(ctypes.sizeof(Config), hidden, num_experts, top_k, num_shared, inter, max_tokens, num_layers, flags)
    h = Handle()
    _check(lib().moe_decode_create(ctypes.byref(cfg), _stream(stream) if stream != 0 else None, ctypes.byref(h)))
    h.sizes = dict(H=hidden, E=num_experts, k=top_k, S=num_shared, I=inter, T=max_tokens, L=num_layers)
    return h


def moe_decode_set_layer(handle, layer: int, router, w13, w13_s, w2, w2_s, stream=None) -> None:
    z = getattr(handle, "sizes", None)
    H, E, S, I = (None,) * 4 if z is None else (z["H"], z["E"], z["S"], z["I"])
    n = None if z is None else E + S

    def nbytes(f):
        return None if z is None else f()

    d = LayerDesc(_tensor(router, DT_BF16, "router", nbytes(lambda: E * H * 2)),
                  _tensor(w13, DT_E2M1X2, "w13", nbytes(lambda: n * I * H)),
                  _tensor(w13_s, DT_E8M0, "w13_s", nbytes(lambda: n * 2 * I * H // 32)),
                  _tensor(w2, DT_E2M1X2, "w2", nbytes(lambda: n * H * I // 2)),
                  _tensor(w2_s, DT_E8M0, "w2_s", nbytes(lambda: n * H * I // 32)))
    _check(lib().moe_decode_set_layer(handle, layer, ctypes.byref(d), _stream(stream)))


def moe_decode_run(handle, x, num_tokens: int | None = None, x_out=None, y=None, topk_ids=None, topk_w=None,
                   x_trace=None, x_scale=None, x_codes=None, stream=None) -> None:
    import torch
    T = x.shape[0] if num_tokens is None else num_tokens
    z = getattr(handle, "sizes", None)
    if z is not None:
        H, L, k = z["H"], z["L"], z["k"]
        if x.dtype != torch.bfloat16:
            raise ValueError(f"x: dtype {x.dtype}, expected torch.bfloat16")
        if not 1 <= T <= z["T"] or x.numel() < T * H:
            raise ValueError(f"x: {tuple(x.shape)} holds fewer than {T} tokens of {H}")
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("x: not a contiguous GPU tensor")
        for t, name, dt, nbytes in ((x_out, "x_out", torch.bfloat16, T * H * 2), (y, "y", torch.float32, T * H * 4),
                                    (topk_ids, "topk_ids", torch.int32, L * T * k * 4),
                                    (topk_w, "topk_w", torch.float32, L * T * k * 4),
                                    (x_trace, "x_trace", torch.bfloat16, L * T * H * 2),
                                    (x_scale, "x_scale", torch.float32, L * T * 4),
                                    (x_codes, "x_codes", torch.uint8, L * T * H)):
            if t is not None:
                if t.dtype != dt:
                    raise ValueError(f"{name}: dtype {t.dtype}, expected {dt}")
                _check_buffer(t, name, nbytes)
    o = Outputs(ctypes.sizeof(Outputs), _ptr(x_out), _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(x_trace),
                _ptr(x_scale), _ptr(x_codes))
    _check(lib().moe_decode_run(handle, _ptr(x), T, ctypes.byref(o), _stream(stream)))


def moe_decode_query(handle) -> dict:
    info = Info()
    info.struct_size = ctypes.sizeof(Info)
    _check(lib().moe_decode_query(handle, ctypes.byref(info)))
    return {"variant": info.variant.decode(), "weight_bytes": info.weight_bytes,
            "workspace_bytes": info.workspace_bytes, "bytes_per_layer_t1": info.bytes_per_layer_t1,
            "layers_set": info.layers_set, "jit_from_cache": bool(info.jit_from_cache),
            "jit_compile_ms": info.jit_compile_ms, "jit_code_object": info.jit_code_object.decode()}


def moe_decode_check(handle) -> None:
    """Waits for the device; raises MoeError if a run of this handle was aborted."""
    _check(lib().moe_decode_check(handle))


def moe_decode_destroy(handle) -> None:
    _check(lib().moe_decode_destroy(handle))


def moe_decode_timing_enable(handle, max_runs: int, mode: int = 0) -> None:
    """mode 0: kernels launched one by one between kernel-stamped events; mode 1: graph replays with
    per-workgroup wall-clock stamps (spans and gaps)."""
    _check(lib().moe_decode_timing_enable(handle, max_runs, mode))


def moe_decode_timing_read(handle) -> dict:
    t = Timing()
    t.struct_size = ctypes.sizeof(Timing)
    _check(lib().moe_decode_timing_read(handle, ctypes.byref(t)))
    return {"runs": t.runs, "mode": t.mode,
            **{c: {"launches": t.launches[i], "total_ms": t.total_ms[i], "gap_launches": t.gap_launches[i],
                   "gap_ms": t.gap_ms[i]} for i, c in enumerate(TIMING_CLASSES)}}


def fp8_head_create(w, row_scale, stream=None) -> ctypes.c_void_p:
    wt = w[0] if isinstance(w, tuple) else w
    vocab, hidden = wt.shape
    h = Handle()
    _check(lib().fp8_head_create(vocab, hidden, _tensor(w, DT_E4M3, "w", vocab * hidden),
                                 _tensor(row_scale, DT_FP32, "row_scale", vocab * 4), _stream(stream), ctypes.byref(h)))
    h.sizes = dict(V=vocab, H=hidden)
    return h


def bf16_head_create(w, stream=None) -> ctypes.c_void_p:
    """The BF16 head (w torch bfloat16 [V][H], device); run and free it with fp8_head_run and
    fp8_head_destroy."""
    vocab, hidden = w.shape
    h = Handle()
    _check(lib().bf16_head_create(vocab, hidden, _tensor(w, DT_BF16, "w", vocab * hidden * 2), _stream(stream),
                                  ctypes.byref(h)))
    h.sizes = dict(V=vocab, H=hidden)
    return h


def _check_head_io(handle, x, T, outs):
    import torch
    z = getattr(handle, "sizes", None)
    if z is None:
        return
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.numel() < T * z["H"]:
        raise ValueError(f"x: needs a contiguous bfloat16 GPU tensor of {T} x {z['H']}")
    for t, name, dt, nbytes in outs:
        if t is not None:
            if t.dtype != dt:
                raise ValueError(f"{name}: dtype {t.dtype}, expected {dt}")
            _check_buffer(t, name, nbytes(z))


def fp8_head_run(handle, x, argmax, logits=None, num_tokens: int | None = None, stream=None) -> None:
    import torch
    T = x.shape[0] if num_tokens is None else num_tokens
    _check_head_io(handle, x, T, ((argmax, "argmax", torch.int32, lambda z: T * 4),
                                  (logits, "logits", torch.float32, lambda z: T * z["V"] * 4)))
    _check(lib().fp8_head_run(handle, _ptr(x), T, _ptr(logits), _ptr(argmax), _stream(stream)))


def fp8_head_verify(handle, x, draft, argmax, accept, stream=None) -> None:
    """Head of a verify step (x [T][H] bf16, draft int32 [T-1], argmax int32 [T], accept int32 [1],
    all on the device): argmax and the number of accepted drafts; enqueues only."""
    import torch
    T = x.shape[0]
    _check_head_io(handle, x, T, ((draft, "draft", torch.int32, lambda z: (T - 1) * 4),
                                  (argmax, "argmax", torch.int32, lambda z: T * 4),
                                  (accept, "accept", torch.int32, lambda z: 4)))
    _check(lib().fp8_head_verify(handle, _ptr(x), T, _ptr(draft), _ptr(argmax), _ptr(accept), _stream(stream)))


def fp8_head_run_noalloc(w, row_scale, x, argmax, logits=None, num_tokens: int | None = None, stream=None) -> None:
    """The FP8 head on the caller's row-major E4M3 weights w [V][H] (uint8 or float8_e4m3fn) and row
    scales [V] (float32), without a handle and without any device allocation; enqueues only."""
    import torch
    vocab, hidden = w.shape
    T = x.shape[0] if num_tokens is None else num_tokens
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.numel() < T * hidden:
        raise ValueError(f"x: needs a contiguous bfloat16 GPU tensor of {T} x {hidden}")
    for t, name, dt, nbytes in ((argmax, "argmax", torch.int32, T * 4), (logits, "logits", torch.float32, T * vocab * 4)):
        if t is not None:
            if t.dtype != dt:
                raise ValueError(f"{name}: dtype {t.dtype}, expected {dt}")
            _check_buffer(t, name, nbytes)
    _check(lib().fp8_head_run_noalloc(vocab, hidden, _tensor(w, DT_E4M3, "w", vocab * hidden),
                                      _tensor(row_scale, DT_FP32, "row_scale", vocab * 4), _ptr(x), T, _ptr(logits),
                                      _ptr(argmax), _stream(stream)))


def moe_probe_stream_read(src, out, grid: int, stream=None) -> None:
    """Streaming read of the whole device tensor src (the practical HBM read ceiling); out: uint32
    [grid] on the device.  Enqueues only."""
    _check(lib().moe_probe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(out), grid,
                                       _stream(stream)))


def fp8_head_destroy(handle) -> None:
    _check(lib().fp8_head_destroy(handle))


def fp8_head_quantize(w, codes, scales, stream=None) -> None:
    """Per-row E4M3 quantisation of w (torch bf16 or float32 [rows][cols], device) into codes
    (uint8 [rows][cols]) and scales (float32 [rows]); enqueues only."""
    import torch
    rows, cols = w.shape
    _check_buffer(codes, "codes", rows * cols)
    _check_buffer(scales, "scales", rows * 4)
    if scales.dtype != torch.float32:
        raise ValueError(f"scales: dtype {scales.dtype}, expected torch.float32")
    _check(lib().fp8_head_quantize(rows, cols, _tensor(w, -1, "w", rows * cols * w.element_size()), _ptr(codes),
                                   _ptr(scales), _stream(stream)))
