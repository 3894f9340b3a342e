"""GPU parity of the MoE decode path (C ABI) against the CPU oracle.

Criteria: expert ids bit-exact, routing weights within 1e-5, per-token FP8 activation scale and
codes bit-exact, y within 2e-3 normwise per token.  Seeds are chosen (tests/golden/manifest.json,
or a margin search with the oracle) so that the ordered top-k is unique under any fp32 summation.
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemv_amd as moe
import oracle
import synth
from gpu_cases import (MANIFEST, VARIANTS, DeviceLayer, bf16_bits, check_layer, create, dev, elementwise_rel_err,
                       margin_attempt, normwise_err, run_layer, set_variant, to_dev_u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True, params=sorted(VARIANTS))
def variant(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    print(f"kernels: {request.param}", flush=True)
    set_variant(request.param)
    yield request.param
    set_variant("aot")


def _layer_case(shape, seed, x, layer_obj=None, handle=None):
    lay = layer_obj or DeviceLayer(shape, seed)
    h = handle or create(shape)
    if handle is None:
        lay.set_into(h, 0)
    gpu = run_layer(h, shape, x)
    ro = oracle.route(shape, lay.router_host, x)
    ref_y, ref_tr = oracle.moe_layer(shape, lay.router_host, lay.oracle_experts(ro["ids"]), x)
    if handle is None:
        moe.moe_decode_destroy(h)
    return gpu, ref_y, ref_tr


def test_device_generator_matches_host():
    for shape, e in ((synth.TINY, 3), (synth.FLASH, 512)):
        lay = DeviceLayer(shape, 7)
        host = synth.expert(shape, 7, 0, e)
        for name in ("w13", "w13_s", "w2", "w2_s"):
            assert (getattr(lay, name)[e].cpu().numpy() == host[name]).all(), (shape, name)


@pytest.mark.parametrize("case,T", [("tiny", 1), ("tiny_t4", 4)])
def test_tiny_layer_manifest(case, T):
    m = MANIFEST[case]
    shape = synth.TINY
    x = synth.tokens(shape.hidden, m["seed"], T, m["x_attempt"])
    gpu, ref_y, ref_tr = _layer_case(shape, m["seed"], x)
    assert gpu["topk_ids"][0].tolist() == m["ids"]
    check_layer(shape, gpu, ref_y, ref_tr)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_tiny_layer_random_seeds(T):
    shape = synth.TINY
    for seed in range(20, 26):
        lay = DeviceLayer(shape, seed)
        h = create(shape)
        lay.set_into(h, 0)
        a, x = margin_attempt(shape, lay.router_host, seed, T)
        gpu, ref_y, ref_tr = _layer_case(shape, seed, x, lay, h)
        check_layer(shape, gpu, ref_y, ref_tr)
        moe.moe_decode_destroy(h)


def test_tiny_shapes_without_shared_and_k1():
    for shape in (synth.Shape(256, 16, 1, 0, 64), synth.Shape(512, 64, 4, 1, 128), synth.Shape(256, 16, 2, 0, 256)):
        lay = DeviceLayer(shape, 31)
        a, x = margin_attempt(shape, lay.router_host, 31, 3)
        gpu, ref_y, ref_tr = _layer_case(shape, 31, x, lay)
        check_layer(shape, gpu, ref_y, ref_tr)


# One shape per kernel geometry accepted besides the tiny and flash ones: router and gate/up
# workgroups of 2, 3, 4 and 5 waves with 8 or 4 MX blocks per lane; down splits of 8 x 1, 4 x 1,
# 2 x 1 and 8 x 3 lanes x blocks, one or two down workgroups per CU at 3-4 tokens; router grids
# whose last workgroup holds fewer experts than waves; no shared expert.
MID_SHAPES = [synth.Shape(1024, 128, 4, 1, 256), synth.Shape(1536, 200, 6, 1, 128), synth.Shape(2048, 256, 8, 1, 768),
              synth.Shape(1280, 128, 8, 0, 64), synth.Shape(768, 40, 3, 1, 256)]


@pytest.mark.parametrize("shape", MID_SHAPES,
                         ids=lambda s: f"H{s.hidden}-E{s.num_experts}-k{s.top_k}-S{s.num_shared}-I{s.inter}")
def test_mid_shapes_every_geometry(shape):
    """Each geometry at 1, 2, 3 and 4 tokens through one handle: ids exact, weights, activation
    scale and codes, and y against the oracle."""
    lay = DeviceLayer(shape, 41)
    h = create(shape)
    lay.set_into(h, 0)
    for T in (1, 2, 3, 4):
        _, x = margin_attempt(shape, lay.router_host, 41, T)
        print(f"shape {shape} T={T}", flush=True)
        gpu, ref_y, ref_tr = _layer_case(shape, 41, x, lay, h)
        check_layer(shape, gpu, ref_y, ref_tr)
    moe.moe_decode_destroy(h)


def _wide_range_attempt(shape, router_host, seed, T):
    for a in range(1000):
        x = synth.tokens_wide_range(shape.hidden, seed, T, a)
        ro = oracle.route(shape, router_host, x)
        if all(oracle.topk_margin_ok(ro["logits"][t], ro["bounds"][t], shape.top_k) for t in range(T)):
            return x
    raise RuntimeError("no wide-range attempt with a routing margin")


@pytest.mark.parametrize("shape,T", [(synth.TINY, 1), (synth.TINY, 4), (synth.FLASH, 4)], ids=["tiny-1", "tiny-4",
                                                                                                   "flash-4"])
def test_wide_range_blocks(shape, T):
    """Every block of 32 inputs holds one code of 448 and 31 codes between 2^-3 and 2^-2: a block dot
    product that kept only 14 bits below its largest activation would drop the low bits of the small
    codes (the scaled E2M1 x E4M3 MFMA of gfx950 does), and the FP8 requantisation of h would turn
    those gate/up errors into code changes that move y beyond the tolerance (about 2.6 changed h
    codes per token on the tiny layer)."""
    for seed in ((20, 21, 22, 23) if shape is synth.TINY else (3,)):
        lay = DeviceLayer(shape, seed)
        h = create(shape)
        lay.set_into(h, 0)
        x = _wide_range_attempt(shape, lay.router_host, seed, T)
        gpu, ref_y, ref_tr = _layer_case(shape, seed, x, lay, h)
        err = check_layer(shape, gpu, ref_y, ref_tr)
        print(f"wide-range seed {seed} T={T}: normwise y error {err}")
        moe.moe_decode_destroy(h)


def test_zero_input_gives_zero_output():
    shape = synth.TINY
    lay = DeviceLayer(shape, 5)
    h = create(shape)
    lay.set_into(h, 0)
    gpu = run_layer(h, shape, np.zeros((2, shape.hidden), dtype=np.uint16))
    moe.moe_decode_destroy(h)
    assert (gpu["y"] == 0).all()
    assert (gpu["topk_ids"][0] == np.arange(shape.top_k)[None, :]).all()
    assert (gpu["topk_w"][0] == 1.0 / shape.top_k).all()
    assert (gpu["x_scale"][0] == 1.0).all() and (gpu["x_codes"][0] == 0).all()


@pytest.fixture(scope="module")
def flash_t1(variant):
    m = MANIFEST["layer_t1"]
    shape = synth.FLASH
    lay = DeviceLayer(shape, m["seed"])
    h = create(shape)
    lay.set_into(h, 0)
    yield shape, lay, h, m
    moe.moe_decode_destroy(h)


def test_flash_layer_t1(flash_t1):
    shape, lay, h, m = flash_t1
    x = synth.tokens(shape.hidden, m["seed"], 1, m["x_attempt"])
    gpu, ref_y, ref_tr = _layer_case(shape, m["seed"], x, lay, h)
    assert gpu["topk_ids"][0].tolist() == m["ids"]
    err = check_layer(shape, gpu, ref_y, ref_tr)
    print(f"flash T=1 normwise y error {err}; elementwise {elementwise_rel_err(gpu['y'], ref_y)}")


def test_flash_layer_t4_disjoint():
    m = MANIFEST["layer_t4"]
    shape = synth.FLASH
    lay = DeviceLayer(shape, m["seed"])
    h = create(shape)
    lay.set_into(h, 0)
    x = synth.tokens(shape.hidden, m["seed"], 4, m["x_attempt"])
    gpu, ref_y, ref_tr = _layer_case(shape, m["seed"], x, lay, h)
    assert gpu["topk_ids"][0].tolist() == m["ids"]
    assert len(set(np.asarray(m["ids"]).reshape(-1).tolist())) == 32
    err = check_layer(shape, gpu, ref_y, ref_tr)
    print(f"flash T=4 normwise y error {err}; elementwise {elementwise_rel_err(gpu['y'], ref_y)}")
    # bit-identical on repeat (fixed-order, atomic-free combine)
    again = run_layer(h, shape, x)
    assert (again["y"] == gpu["y"]).all()
    moe.moe_decode_destroy(h)


@pytest.mark.parametrize("T", [2, 3, 4])
def test_flash_layer_overlapping_routing(flash_t1, T):
    """Verify step whose tokens share routed experts (correlated tokens): every distinct expert is
    read once for all of its tokens, and each token's combine still matches the oracle."""
    shape, lay, h, m = flash_t1
    a, x = margin_attempt(shape, lay.router_host, 11, T, rho=0.9)
    gpu = run_layer(h, shape, x)
    ro = oracle.route(shape, lay.router_host, x)
    ref_y, ref_tr = oracle.moe_layer(shape, lay.router_host, lay.oracle_experts(ro["ids"]), x)
    distinct = len(set(ro["ids"].reshape(-1).tolist()))
    err = check_layer(shape, gpu, ref_y, ref_tr)
    print(f"flash T={T} overlapping routing: attempt {a}, {distinct} distinct routed experts, normwise y error {err}")


def test_flash_token_independence(flash_t1):
    shape, lay, h, m = flash_t1
    a, x = margin_attempt(shape, lay.router_host, m["seed"], 4, start=500)
    g4 = run_layer(h, shape, x)
    for t in range(4):
        g1 = run_layer(h, shape, x[t:t + 1])
        assert (g1["topk_ids"][0, 0] == g4["topk_ids"][0, t]).all()
        assert (g1["x_codes"][0, 0] == g4["x_codes"][0, t]).all()
        assert normwise_err(g1["y"][0], g4["y"][t]) <= 1e-5


def test_dtype_tag_mismatch_is_an_error(flash_t1):
    shape, lay, h, m = flash_t1
    with pytest.raises(moe.MoeError) as ei:
        # FP8 bytes presented where bf16 router weights belong: the pages' silent-fallback trap
        moe.moe_decode_set_layer(h, 0, (lay.router, moe.DT_E4M3), lay.w13, lay.w13_s, lay.w2, lay.w2_s)
    assert ei.value.status == -3
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_decode_set_layer(h, 0, lay.router, lay.w13, (lay.w13_s, moe.DT_E2M1X2), lay.w2, lay.w2_s)
    assert ei.value.status == -3


def test_run_before_set_is_a_state_error():
    shape = synth.TINY
    h = create(shape, num_layers=2)
    lay = DeviceLayer(shape, 1)
    lay.set_into(h, 0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_decode_run(h, to_dev_u16(np.zeros((1, shape.hidden), dtype=np.uint16)), 1)
    assert ei.value.status == -7
    info = moe.moe_decode_query(h)
    assert info["layers_set"] == 1
    moe.moe_decode_destroy(h)


def test_query_reports_variant_and_bytes(flash_t1, variant):
    shape, lay, h, m = flash_t1
    info = moe.moe_decode_query(h)
    tags = info["variant"].split("-")[5:]
    assert info["variant"].startswith("gfx950-3k")
    assert ("jit" in tags) == (variant == "jit") and ("mfma" in tags) == (variant == "mfma")
    assert ("flash" in tags) == (variant in ("aot", "mfma"))  # the build with the flash shape folded in
    assert info["bytes_per_layer_t1"] == 30_822_400


def _extreme_scales(w13, w13_s, w2, w2_s, I, xp):
    """Crafted E8M0 bytes on every expert (xp: numpy or torch; arrays [experts][rows][...] or one
    expert's [rows][...] when given 3-D / 2-D views).  Down rows 0-7: scale byte 0 (2^-127, an fp32
    subnormal); rows 8-15: byte 1 (2^-126); rows 16-23: byte 127 (1.0); rows 24-31: byte 254 (2^127) on
    all-zero codes, so a decode of 254 to anything but a finite value would turn 0 into NaN; row 32,
    block 0: byte 255 (NaN).  Gate rows 4-7: byte 254 on all-zero codes; gate rows 0-1, first four
    blocks: byte 0."""
    w2_s[..., 0:8, :] = 0
    w2_s[..., 8:16, :] = 1
    w2_s[..., 16:24, :] = 127
    w2_s[..., 24:32, :] = 254
    w2[..., 24:32, :] = 0
    w2_s[..., 32, 0] = 255
    w13_s[..., 4:8, :] = 254
    w13[..., 4:8, :] = 0
    w13_s[..., 0:2, 0:4] = 0


@pytest.mark.parametrize("shape", [synth.Shape(256, 16, 1, 0, 64), synth.Shape(256, 16, 2, 1, 64)],
                         ids=["k1_no_shared", "k2_shared"])
def test_e8m0_extreme_scale_bytes(shape):
    """E8M0 bytes 0 (2^-127), 1, 127, 254 (2^127) and 255 (NaN) decode as OCP MX defines them:
    NaN reaches exactly the outputs it reaches in the oracle, the subnormal scale is not flushed
    (rows whose every block has byte 0 or 1 match the oracle to 2e-3 of their own magnitude) and
    byte 254 on zero codes contributes 0, not NaN."""
    lay = DeviceLayer(shape, 41)
    _extreme_scales(lay.w13, lay.w13_s, lay.w2, lay.w2_s, shape.inter, torch)
    torch.cuda.synchronize()
    h = create(shape)
    lay.set_into(h, 0)
    a, x = margin_attempt(shape, lay.router_host, 41, 2)
    gpu = run_layer(h, shape, x)
    moe.moe_decode_destroy(h)
    ro = oracle.route(shape, lay.router_host, x)
    experts = lay.oracle_experts(ro["ids"])
    for e in experts.values():
        _extreme_scales(e["w13"], e["w13_s"], e["w2"], e["w2_s"], shape.inter, np)
    ref_y, ref_tr = oracle.moe_layer(shape, lay.router_host, experts, x)
    assert (gpu["topk_ids"][0] == ref_tr["ids"]).all()
    assert (np.isnan(gpu["y"]) == np.isnan(ref_y)).all(), np.argwhere(np.isnan(gpu["y"]) != np.isnan(ref_y))[:8]
    assert np.isnan(ref_y[:, 32]).all() and not np.isnan(np.delete(ref_y, 32, axis=1)).any()
    for rows in (slice(0, 8), slice(8, 16), slice(16, 24)):
        g, r = gpu["y"][:, rows].astype(np.float64), ref_y[:, rows].astype(np.float64)
        mag = np.abs(r).max(axis=1, keepdims=True)
        assert (mag > 0).all() and (np.abs(g - r) <= Y_TOL_ROWS * mag).all(), (rows, g, r)
    assert (ref_y[:, 24:32] == ref_y[:, 24:32]).all()  # finite
    ok = ~np.isnan(ref_y)
    err = np.abs(gpu["y"][ok] - ref_y[ok]).max() / np.abs(ref_y[ok]).max()
    assert err <= 2e-3


Y_TOL_ROWS = 2e-3


def test_binding_derives_dtype_tags_from_tensors(flash_t1):
    """A float32 router with the right byte count, and E4M3 codes handed over as bf16, are refused by
    the library's tag check (the binding tags each tensor from its own dtype); a tensor of the wrong
    size is refused by the binding before any device work."""
    shape, lay, h, m = flash_t1
    f32_router = lay.router.view(torch.float32)  # same bytes, float32 dtype
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_decode_set_layer(h, 0, f32_router, lay.w13, lay.w13_s, lay.w2, lay.w2_s)
    assert ei.value.status == -3
    with pytest.raises(ValueError):
        moe.moe_decode_set_layer(h, 0, lay.router[:-1], lay.w13, lay.w13_s, lay.w2, lay.w2_s)
    # E4M3 head weights handed over as bf16 values: refused (tag BF16 in an E4M3 slot, or a size
    # that is not one byte per weight)
    w_bf16 = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    scales = torch.ones((64,), dtype=torch.float32, device="cuda")
    with pytest.raises((moe.MoeError, ValueError)):
        moe.fp8_head_create(w_bf16, scales)
    # the same bytes presented as one byte per weight but tagged from the bf16 tensor they came from
    w_bytes = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.fp8_head_create((w_bytes, moe._dtype_tag(w_bf16, moe.DT_E4M3)), scales)
    assert ei.value.status == -3


def test_graph_replay_timing_record(flash_t1):
    """Timing mode 1 (graph replays with per-workgroup wall-clock stamps): one span per kernel and
    layer of every recorded run, gaps for every kernel after the first, and the record's spans and
    gaps add up to no more than the wall time of the runs; the outputs are unchanged."""
    shape, lay, h, m = flash_t1
    x = synth.tokens(shape.hidden, m["seed"], 1, m["x_attempt"])
    ref = run_layer(h, shape, x)
    moe.moe_decode_timing_enable(h, 3, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        got = run_layer(h, shape, x)
    e1.record()
    torch.cuda.synchronize()
    t = moe.moe_decode_timing_read(h)
    moe.moe_decode_timing_enable(h, 0)
    assert t["mode"] == 1 and t["runs"] == 3
    for c in ("router", "gateup", "down"):
        assert t[c]["launches"] == 3 and t[c]["total_ms"] > 0, (c, t[c])
    assert t["router"]["gap_launches"] == 0 and t["gateup"]["gap_launches"] == 3 and t["down"]["gap_launches"] == 3
    assert t["input"]["launches"] == 0 and t["requant"]["launches"] == 0
    recorded = sum(t[c]["total_ms"] + t[c]["gap_ms"] for c in moe.TIMING_CLASSES)
    assert 0 < recorded <= e0.elapsed_time(e1)
    assert (got["y"] == ref["y"]).all()


def _fixed_outputs(shape, T):
    """One set of output buffers; runs that pass the same set (and x, T) replay one captured graph."""
    H, k = shape.hidden, shape.top_k
    f32 = dict(dtype=torch.float32, device=dev())
    return {"y": torch.full((T, H), float("nan"), **f32),
            "x_out": torch.empty((T, H), dtype=torch.bfloat16, device=dev()),
            "topk_ids": torch.full((1, T, k), -1, dtype=torch.int32, device=dev()),
            "topk_w": torch.full((1, T, k), float("nan"), **f32),
            "x_trace": torch.empty((1, T, H), dtype=torch.bfloat16, device=dev()),
            "x_scale": torch.full((1, T), float("nan"), **f32),
            "x_codes": torch.empty((1, T, H), dtype=torch.uint8, device=dev())}


def _read(out):
    res = {n: t.cpu().numpy() for n, t in out.items() if t.dtype != torch.bfloat16}
    res["x_out"] = bf16_bits(out["x_out"])
    res["x_trace"] = bf16_bits(out["x_trace"])
    return res


def _assert_same(a, b, what):
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), f"{what}: {n} differs"


def test_direct_launch_equals_graph_replay():
    """MOE_F_DIRECT_LAUNCH (the kernels enqueued at every run) and the default captured-graph replay
    give bit-identical outputs, tiny and flash layers at 1-4 tokens."""
    for shape, seed in ((synth.TINY, 7), (synth.FLASH, 7)):
        lay = DeviceLayer(shape, seed)
        hg, hd = create(shape), create(shape, flags=moe.F_DIRECT_LAUNCH)
        lay.set_into(hg, 0)
        lay.set_into(hd, 0)
        for T in (1, 2, 3, 4):
            _, x = margin_attempt(shape, lay.router_host, seed, T)
            print(f"shape {shape} T={T}", flush=True)
            _assert_same(run_layer(hg, shape, x), run_layer(hd, shape, x), f"{shape} T={T}")
        moe.moe_decode_destroy(hg)
        moe.moe_decode_destroy(hd)


def test_graph_replay_picks_up_new_inputs_and_weights():
    """A graph is captured per (x, T, outputs) and holds pointers: replays with new contents of x, and
    after set_layer has replaced the layer's weights, compute the new results (checked against the
    oracle each time)."""
    shape, T = synth.TINY, 2
    la, lb = DeviceLayer(shape, 50), DeviceLayer(shape, 51)
    h = create(shape)
    la.set_into(h, 0)
    a1, x1 = margin_attempt(shape, la.router_host, 50, T)
    _, x2 = margin_attempt(shape, la.router_host, 50, T, start=a1 + 1)
    _, x3 = margin_attempt(shape, lb.router_host, 51, T)
    xd = to_dev_u16(x1)
    out = _fixed_outputs(shape, T)

    def run_and_check(lay, x):
        moe.moe_decode_run(h, xd, T, **out)
        torch.cuda.synchronize()
        moe.moe_decode_check(h)
        ro = oracle.route(shape, lay.router_host, x)
        ref_y, ref_tr = oracle.moe_layer(shape, lay.router_host, lay.oracle_experts(ro["ids"]), x)
        check_layer(shape, _read(out), ref_y, ref_tr)

    run_and_check(la, x1)  # captured
    run_and_check(la, x1)  # replayed
    xd.copy_(to_dev_u16(x2))
    run_and_check(la, x2)  # same graph, new x
    lb.set_into(h, 0)
    xd.copy_(to_dev_u16(x3))
    run_and_check(lb, x3)  # same graph, new weights
    moe.moe_decode_destroy(h)


def test_graph_cache_overflow_with_runs_in_flight():
    """Twenty distinct output sets enqueued back to back with no host wait: the 17th call frees the
    16 captured graphs while their launches may still be queued.  Every output equals the
    direct-launch result, and so do re-captured runs of the first sets."""
    shape = synth.TINY
    lay = DeviceLayer(shape, 52)
    h, hd = create(shape), create(shape, flags=moe.F_DIRECT_LAUNCH)
    lay.set_into(h, 0)
    lay.set_into(hd, 0)
    _, x = margin_attempt(shape, lay.router_host, 52, 1)
    ref = run_layer(hd, shape, x)
    xd = to_dev_u16(x)
    outs = [_fixed_outputs(shape, 1) for _ in range(20)]
    for o in outs:
        moe.moe_decode_run(h, xd, 1, **o)
    torch.cuda.synchronize()
    moe.moe_decode_check(h)
    for i, o in enumerate(outs):
        _assert_same(_read(o), ref, f"output set {i}")
    for o in outs[:3]:
        for t in o.values():
            t.zero_()
        moe.moe_decode_run(h, xd, 1, **o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs[:3]):
        _assert_same(_read(o), ref, f"re-captured output set {i}")
    moe.moe_decode_destroy(h)
    moe.moe_decode_destroy(hd)


def test_two_handles_on_two_streams_do_not_interfere():
    """Handles share no device state (workspace, routing list, arrival ticket, graphs): two handles
    with different weights, run three times each on two streams with no host wait between the
    calls, give bit for bit the outputs each gives alone (4 tokens: the ticket form)."""
    shape, T = synth.FLASH, 4
    la, lb = DeviceLayer(shape, 60), DeviceLayer(shape, 61)
    ha, hb = create(shape), create(shape)
    la.set_into(ha, 0)
    lb.set_into(hb, 0)
    _, xa = margin_attempt(shape, la.router_host, 60, T)
    _, xb = margin_attempt(shape, lb.router_host, 61, T)
    ref_a, ref_b = run_layer(ha, shape, xa), run_layer(hb, shape, xb)
    xda, xdb = to_dev_u16(xa), to_dev_u16(xb)
    outs_a = [_fixed_outputs(shape, T) for _ in range(3)]
    outs_b = [_fixed_outputs(shape, T) for _ in range(3)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        moe.moe_decode_run(ha, xda, T, stream=sa, **oa)
        moe.moe_decode_run(hb, xdb, T, stream=sb, **ob)
    torch.cuda.synchronize()
    moe.moe_decode_check(ha)
    moe.moe_decode_check(hb)
    for i in range(3):
        _assert_same(_read(outs_a[i]), ref_a, f"handle a, run {i}")
        _assert_same(_read(outs_b[i]), ref_b, f"handle b, run {i}")
    moe.moe_decode_destroy(ha)
    moe.moe_decode_destroy(hb)
