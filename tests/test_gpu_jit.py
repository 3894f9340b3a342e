"""Run-time compilation of the MoE kernels for one layer shape (MOE_F_JIT), through the C ABI: the
first create compiles and fills the on-disk cache, a second create with the same shape loads the
code object without compiling, a different shape gets its own entry, and the compiled kernels give
the ahead-of-time kernels' outputs bit for bit (the same arithmetic, with the shape as constants).
The parity of the JIT kernels against the oracle is covered by the MoE and stack tests, which run on
both builds."""
import os

import numpy as np
import pytest
import torch

import mxfp4_expert_gemv_amd as moe
import synth
from gpu_cases import MANIFEST, DeviceLayer, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cache_dir(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = str(tmp_path_factory.mktemp("jit_cache"))
    old = os.environ.get("MOE_JIT_CACHE_DIR")
    os.environ["MOE_JIT_CACHE_DIR"] = d
    yield d
    if old is None:
        del os.environ["MOE_JIT_CACHE_DIR"]
    else:
        os.environ["MOE_JIT_CACHE_DIR"] = old


def _create(shape, flags):
    return moe.moe_decode_create(shape.hidden, shape.num_experts, shape.top_k, shape.num_shared, shape.inter, 4, 1,
                                 flags)


def test_compile_then_cache_hit(cache_dir):
    shape = synth.FLASH
    h1 = _create(shape, moe.F_JIT)
    i1 = moe.moe_decode_query(h1)
    moe.moe_decode_destroy(h1)
    print(f"first create: compiled in {i1['jit_compile_ms']:.0f} ms into {i1['jit_code_object']}", flush=True)
    assert not i1["jit_from_cache"] and i1["jit_compile_ms"] > 0
    assert i1["jit_code_object"].startswith(cache_dir) and os.path.exists(i1["jit_code_object"])
    h2 = _create(shape, moe.F_JIT)
    i2 = moe.moe_decode_query(h2)
    moe.moe_decode_destroy(h2)
    assert i2["jit_from_cache"] and i2["jit_compile_ms"] == 0 and i2["jit_code_object"] == i1["jit_code_object"]
    # another shape, or another input normalisation, is another cache entry
    h3 = _create(synth.TINY, moe.F_JIT)
    i3 = moe.moe_decode_query(h3)
    moe.moe_decode_destroy(h3)
    h4 = _create(shape, moe.F_JIT | moe.F_RMSNORM_INPUT)
    i4 = moe.moe_decode_query(h4)
    moe.moe_decode_destroy(h4)
    assert not i3["jit_from_cache"] and not i4["jit_from_cache"]
    assert len({i1["jit_code_object"], i3["jit_code_object"], i4["jit_code_object"]}) == 3


@pytest.mark.parametrize("norm", [0, moe.F_RMSNORM_INPUT], ids=["raw", "rmsnorm"])
@pytest.mark.parametrize("base", [0, moe.F_MFMA], ids=["valu", "mfma"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_jit_kernels_match_the_ahead_of_time_kernels_bit_for_bit(cache_dir, T, base, norm):
    """The run-time compiled kernels, the ahead-of-time build with the flash shape folded in and the
    shape-generic ahead-of-time build compute the same bytes."""
    m = MANIFEST["layer_t4"]
    shape = synth.FLASH
    lay = DeviceLayer(shape, m["seed"])
    x = synth.tokens(shape.hidden, m["seed"], 4, m["x_attempt"])[:T]
    out = {}
    for name, flags in (("aot", base), ("generic", base | moe.F_GENERIC), ("jit", base | moe.F_JIT)):
        h = _create(shape, flags | norm)
        tags = moe.moe_decode_query(h)["variant"].split("-")[5:]
        assert ("flash" in tags) == (name == "aot"), (name, tags)
        lay.set_into(h, 0)
        out[name] = run_layer(h, shape, x)
        moe.moe_decode_destroy(h)
    for other in ("generic", "jit"):
        for k in ("y", "topk_ids", "topk_w", "x_scale", "x_codes"):
            a, b = out["aot"][k], out[other][k]
            assert (a.view(np.uint8) == b.view(np.uint8)).all(), (other, k)


def test_unwritable_cache_still_compiles(cache_dir, monkeypatch):
    """A cache directory that cannot be created only costs a compile: the handle still runs the
    run-time compiled kernels (never the ahead-of-time ones)."""
    monkeypatch.setenv("MOE_JIT_CACHE_DIR", "/proc/no_such_dir/cache")
    h = _create(synth.TINY, moe.F_JIT)
    info = moe.moe_decode_query(h)
    moe.moe_decode_destroy(h)
    assert info["variant"].endswith("-jit") and not info["jit_from_cache"]
