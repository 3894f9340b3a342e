"""Shared helpers of the GPU parity tests: seeded inputs on the device, oracle references, checks.

Inputs come from ``synth`` (the seeded generator both sides consume); expected values come only
from ``oracle``.  The GPU path is reached only through the C ABI binding ``mxfp4_expert_gemv_amd``.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import mxfp4_expert_gemv_amd as moe
import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
MANIFEST = json.load(open(os.path.join(HERE, "golden", "manifest.json")))

# Normwise per-token bound on y: max_j |y_gpu - y_ref| / max_j |y_ref|.
Y_TOL = 2e-3
W_TOL = 1e-5


def dev():
    return torch.device("cuda:0")


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    """uint16 host array (bf16 bits) -> device bf16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceLayer:
    """Canonical device tensors of one layer: router bf16 [E][H] and the MXFP4 tensors of all
    E+S experts, generated on the device by the integer twin of the host generator."""

    def __init__(self, shape: synth.Shape, seed: int, layer: int = 0, router_attempt: int = 0):
        self.shape, self.seed, self.layer = shape, seed, layer
        self.router_host = synth.router(shape, seed, layer, router_attempt)
        self.router = to_dev_u16(self.router_host)
        n = shape.num_experts + shape.num_shared
        H, I = shape.hidden, shape.inter
        u8 = dict(dtype=torch.uint8, device=dev())
        self.w13 = torch.empty((n, 2 * I, H // 2), **u8)
        self.w13_s = torch.empty((n, 2 * I, H // 32), **u8)
        self.w2 = torch.empty((n, H, I // 2), **u8)
        self.w2_s = torch.empty((n, H, I // 32), **u8)
        synth.fill_experts_device(self.w13, self.w13_s, self.w2, self.w2_s, shape, seed, layer,
                                  stream=torch.cuda.current_stream().cuda_stream)

    def set_into(self, handle, layer: int | None = None):
        moe.moe_decode_set_layer(handle, self.layer if layer is None else layer, self.router, self.w13, self.w13_s,
                                 self.w2, self.w2_s)

    def oracle_experts(self, ids) -> dict:
        used = sorted(set(int(e) for e in np.asarray(ids).reshape(-1))) + ([self.shape.num_experts]
                                                                           if self.shape.num_shared else [])
        return {e: synth.expert(self.shape, self.seed, self.layer, e) for e in used}


# the kernel builds behind the same calls: compiled ahead of time (default), compiled at run time for
# the handle's shape (MOE_F_JIT), and the gate/up dot products on the scaled matrix cores
# (MOE_F_MFMA); the MoE parity tests run on each
# aot: the ahead-of-time kernels (for the flash layer shape, the build with that shape folded in);
# generic: the shape-generic ahead-of-time kernels on every shape
VARIANTS = {"aot": 0, "generic": moe.F_GENERIC, "jit": moe.F_JIT, "mfma": moe.F_MFMA}
_variant = {"flags": 0}


def set_variant(name: str):
    _variant["flags"] = VARIANTS[name]


def create(shape: synth.Shape, max_tokens: int = 4, num_layers: int = 1, flags: int = 0):
    return moe.moe_decode_create(shape.hidden, shape.num_experts, shape.top_k, shape.num_shared, shape.inter,
                                 max_tokens, num_layers, flags | _variant["flags"])


def run_layer(handle, shape: synth.Shape, x_host: np.ndarray, num_layers: int = 1) -> dict:
    """Runs the handle on bf16 bits x [T][H]; returns every output as numpy."""
    T, H = x_host.shape
    k = shape.top_k
    x = to_dev_u16(x_host)
    f32 = dict(dtype=torch.float32, device=dev())
    out = {"y": torch.full((T, H), float("nan"), **f32),
           "x_out": torch.empty((T, H), dtype=torch.bfloat16, device=dev()),
           "topk_ids": torch.full((num_layers, T, k), -1, dtype=torch.int32, device=dev()),
           "topk_w": torch.full((num_layers, T, k), float("nan"), **f32),
           "x_trace": torch.empty((num_layers, T, H), dtype=torch.bfloat16, device=dev()),
           "x_scale": torch.full((num_layers, T), float("nan"), **f32),
           "x_codes": torch.empty((num_layers, T, H), dtype=torch.uint8, device=dev())}
    moe.moe_decode_run(handle, x, T, **out)
    torch.cuda.synchronize()
    moe.moe_decode_check(handle)  # raises on an asynchronous device error
    res = {n: t.cpu().numpy() for n, t in out.items() if t.dtype != torch.bfloat16}
    res["x_out"] = bf16_bits(out["x_out"])
    res["x_trace"] = bf16_bits(out["x_trace"])
    return res


def normwise_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per token max |y_gpu - y_ref| / max |y_ref| (0 where y_ref is identically 0 and y_gpu too)."""
    y_gpu = y_gpu.astype(np.float64)
    y_ref = y_ref.astype(np.float64)
    num = np.abs(y_gpu - y_ref).max(axis=-1)
    den = np.abs(y_ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def elementwise_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray, floor: float = 1e-3) -> dict:
    """For information: |y_gpu - y_ref| / |y_ref| element by element, over the elements with
    |y_ref| >= floor * max |y_ref| of their token (the elementwise form is ill-posed near zero):
    median, p99 and maximum, and the fraction of elements covered."""
    y_gpu = y_gpu.astype(np.float64)
    y_ref = y_ref.astype(np.float64)
    den = np.abs(y_ref)
    keep = den >= floor * den.max(axis=-1, keepdims=True)
    r = np.abs(y_gpu - y_ref)[keep] / den[keep]
    return {"median": float(np.median(r)), "p99": float(np.percentile(r, 99)), "max": float(r.max()),
            "covered": float(keep.mean())}


def check_layer(shape, gpu: dict, ref_y: np.ndarray, ref_tr: dict, layer: int = 0, check_codes: bool = True):
    """GPU outputs of one layer against the oracle: ids bit-exact, weights within W_TOL, activation
    scale and codes bit-exact, y within Y_TOL normwise."""
    ids = gpu["topk_ids"][layer]
    assert (ids == ref_tr["ids"]).all(), f"ids differ:\n gpu {ids.tolist()}\n ref {ref_tr['ids'].tolist()}"
    assert np.abs(gpu["topk_w"][layer] - ref_tr["w"]).max() <= W_TOL
    if check_codes:
        assert (gpu["x_scale"][layer] == ref_tr["sx"]).all(), (gpu["x_scale"][layer], ref_tr["sx"])
        bad = np.argwhere(gpu["x_codes"][layer] != ref_tr["qx"])
        assert bad.size == 0, f"{len(bad)} activation codes differ, first at {bad[:5].tolist()}"
    err = normwise_err(gpu["y"], ref_y)
    assert (err <= Y_TOL).all(), f"normwise y error {err}"
    return err


def margin_attempt(shape, router_host, seed, T, start=0, need_disjoint=False, rho=None):
    """First x attempt >= start whose routing is well posed under fp32 evaluation.  With rho, the
    tokens are correlated (synth.tokens_correlated) and the attempt must share at least one routed
    expert between tokens."""
    for a in range(start, start + 10000):
        x = synth.tokens(shape.hidden, seed, T, a) if rho is None else synth.tokens_correlated(shape.hidden, seed, T,
                                                                                                rho, a)
        ro = oracle.route(shape, router_host, x)
        ok = all(oracle.topk_margin_ok(ro["logits"][t], ro["bounds"][t], shape.top_k) for t in range(T))
        distinct = len(set(ro["ids"].reshape(-1).tolist()))
        if ok and need_disjoint:
            ok = distinct == ro["ids"].size
        if ok and rho is not None:
            ok = distinct < ro["ids"].size
        if ok:
            return a, x
    raise RuntimeError("no attempt with a routing margin")
