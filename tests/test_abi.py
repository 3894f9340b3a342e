"""The C-ABI library loads without a GPU, exports every function include/moe_decode.h declares,
and validates its arguments before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest

import mxfp4_expert_gemv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared():
        assert hasattr(L, name), name


def _status(cfg_kwargs):
    c = dict(hidden=2560, num_experts=512, top_k=8, num_shared=1, inter=768, max_tokens=4, num_layers=1, flags=0)
    c.update(cfg_kwargs)
    cfg = moe.Config(ctypes.sizeof(moe.Config), *[c[f] for f in ("hidden", "num_experts", "top_k", "num_shared",
                                                                  "inter", "max_tokens", "num_layers", "flags")])
    if "struct_size" in cfg_kwargs:
        cfg.struct_size = cfg_kwargs["struct_size"]
    h = ctypes.c_void_p()
    return moe.lib().moe_decode_create(ctypes.byref(cfg), None, ctypes.byref(h))


@pytest.mark.parametrize("bad,status", [
    ({"struct_size": 4}, -1), ({"hidden": 0}, -1), ({"top_k": 9, "num_experts": 8}, -1),
    ({"hidden": 2500}, -2), ({"hidden": 4096}, -2), ({"num_experts": 1024}, -2), ({"num_experts": 12, "top_k": 2}, -2), ({"top_k": 9}, -2),
    ({"num_shared": 2}, -2), ({"inter": 96}, -2), ({"inter": 1024}, -2), ({"max_tokens": 5}, -2),
    ({"flags": 0x80}, -1),
])
def test_create_rejects_bad_configs_before_any_hip_call(bad, status):
    assert _status(bad) == status
    assert moe.lib().moe_last_error()


def test_valid_config_without_device_is_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _status({}) == -6
    assert _status({"hidden": 256, "num_experts": 16, "top_k": 2, "inter": 64}) == -6


def _header_flags():
    text = open(os.path.join(ROOT, "include", "moe_decode.h")).read()
    return {m.group(1): int(m.group(2), 16) for m in re.finditer(r"#define MOE_F_(\w+) (0x[0-9a-fA-F]+)u", text)}


def test_binding_flags_match_the_header():
    flags = _header_flags()
    assert set(flags) == {"RMSNORM_INPUT", "DIRECT_LAUNCH", "JIT", "MFMA", "GENERIC"}
    for name, value in flags.items():
        assert getattr(moe, "F_" + name) == value, name


def test_every_documented_flag_passes_validation_and_other_bits_are_refused():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    known = 0
    for value in _header_flags().values():
        known |= value
        assert _status({"flags": value}) == -6  # valid: only the missing device stops create
    assert _status({"flags": known}) == -6
    for bit in range(32):
        if not (known >> bit) & 1:
            assert _status({"flags": 1 << bit}) == -1, bit


def test_null_arguments():
    L = moe.lib()
    assert L.moe_decode_create(None, None, None) == -1
    assert L.moe_decode_set_layer(None, 0, None, None) == -1
    assert L.moe_decode_run(None, None, 1, None, None) == -1
    assert L.moe_decode_query(None, None) == -1
    assert L.moe_decode_destroy(None) == 0
    assert L.fp8_head_run(None, None, 1, None, None, None) == -1
    assert L.fp8_head_destroy(None) == 0
    t = moe.Tensor(None, moe.DT_E4M3)
    h = ctypes.c_void_p()
    assert L.fp8_head_create(100, 2560, t, moe.Tensor(None, moe.DT_FP32), None, ctypes.byref(h)) == -1
    assert L.moe_status_string(-3) == b"dtype tag mismatch"


def test_head_dtype_tags_checked_before_device():
    L = moe.lib()
    h = ctypes.c_void_p()
    buf = ctypes.create_string_buffer(64)
    addr = (ctypes.addressof(buf) + 15) // 16 * 16
    # bf16-tagged weights where E4M3 is required: the silent-reinterpretation trap is an error
    assert L.fp8_head_create(100, 2560, moe.Tensor(addr, moe.DT_BF16), moe.Tensor(addr, moe.DT_FP32), None,
                             ctypes.byref(h)) == -3
    assert L.fp8_head_create(100, 2560, moe.Tensor(addr, moe.DT_E4M3), moe.Tensor(addr, moe.DT_BF16), None,
                             ctypes.byref(h)) == -3
    assert L.fp8_head_create(100, 2000, moe.Tensor(addr, moe.DT_E4M3), moe.Tensor(addr, moe.DT_FP32), None,
                             ctypes.byref(h)) == -2


def test_head_quantize_arguments_checked_before_device():
    L = moe.lib()
    buf = ctypes.create_string_buffer(64)
    addr = (ctypes.addressof(buf) + 15) // 16 * 16
    ok = moe.Tensor(addr, moe.DT_FP32)
    assert L.fp8_head_quantize(0, 2560, ok, addr, addr, None) == -1
    assert L.fp8_head_quantize(8, 2000, ok, addr, addr, None) == -2
    # E4M3-tagged input: only BF16 or FP32 weights are quantised
    assert L.fp8_head_quantize(8, 2560, moe.Tensor(addr, moe.DT_E4M3), addr, addr, None) == -3
    assert L.fp8_head_quantize(8, 2560, ok, None, addr, None) == -1
    assert L.fp8_head_quantize(8, 2560, ok, addr, None, None) == -1


def test_head_verify_arguments():
    L = moe.lib()
    assert L.fp8_head_verify(None, None, 4, None, None, None, None) == -1
    # every check below fails before the handle would be read, so a stand-in address serves as one
    buf = (ctypes.c_uint8 * 64)()
    addr = (ctypes.addressof(buf) + 15) & ~15
    fake = ctypes.c_void_p(addr)
    for T in (0, 1, 5):  # a verify step scores the current token and 1-3 drafts: 2 <= T <= 4
        assert L.fp8_head_verify(fake, addr, T, addr, addr, addr, None) == -1, T
    assert L.fp8_head_verify(fake, addr, 4, None, addr, addr, None) == -1  # draft is required
    assert L.fp8_head_verify(fake, addr, 4, addr, addr, None, None) == -1  # accept is required
    assert L.fp8_head_verify(fake, addr + 8, 4, addr, addr, addr, None) == -1  # x not 16-byte aligned


def test_binding_tags_tensors_from_their_own_dtype():
    """The binding derives each tag from the tensor's dtype (raw bytes take the slot's byte format),
    so a float32 or bf16 tensor cannot be passed off as FP8 or MXFP4 bytes."""
    import torch
    t = lambda dt: torch.zeros(4, dtype=dt)  # noqa: E731
    assert moe._dtype_tag(t(torch.bfloat16), moe.DT_E2M1X2) == moe.DT_BF16
    assert moe._dtype_tag(t(torch.float32), moe.DT_BF16) == moe.DT_FP32
    assert moe._dtype_tag(t(torch.uint8), moe.DT_E8M0) == moe.DT_E8M0
    assert moe._dtype_tag(t(torch.uint8), moe.DT_E4M3) == moe.DT_E4M3
    assert moe._dtype_tag(t(torch.float8_e4m3fn), moe.DT_E2M1X2) == moe.DT_E4M3
    assert moe._dtype_tag(t(torch.int32), moe.DT_BF16) == -1
    # bf16 weights offered to the FP8 head: the library refuses the tag before any device call
    w = torch.zeros((64, 256), dtype=torch.bfloat16)
    s = torch.ones(64, dtype=torch.float32)
    h = ctypes.c_void_p()
    st = moe.lib().fp8_head_create(64, 256, moe._tensor(w, moe.DT_E4M3), moe._tensor(s, moe.DT_FP32), None,
                                   ctypes.byref(h))
    assert st == -3
    # a float32 router offered where bf16 belongs is tagged FP32 (the set-layer tag check refuses it)
    assert moe._tensor(torch.zeros((16, 256), dtype=torch.float32), moe.DT_BF16).dtype == moe.DT_FP32


def test_binding_refuses_host_and_missized_tensors():
    import torch
    with pytest.raises(ValueError):
        moe._tensor(torch.zeros(16, dtype=torch.uint8), moe.DT_E8M0, "w", 16)  # host memory
