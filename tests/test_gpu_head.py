"""GPU parity of the FP8 LM head (C ABI) against the oracle: logits within the fp32 evaluation
bound the oracle reports, argmax exact (lowest index on ties)."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemv_amd as moe
import oracle
import synth
from gpu_cases import MANIFEST, dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quantised(V, H, seed):
    Wq = np.empty((V, H), dtype=np.uint8)
    s = np.empty(V, dtype=np.float32)
    step = 16384
    for r0 in range(0, V, step):
        n = min(step, V - r0)
        Wq[r0:r0 + n], s[r0:r0 + n] = oracle.head_quantize(synth.head_weights(V, H, seed, r0, n))
    return Wq, s


def _run(Wq, s, x, want_logits=True):
    w = torch.from_numpy(Wq).to(dev())
    sc = torch.from_numpy(s).to(dev())
    h = moe.fp8_head_create(w, sc)
    T = x.shape[0]
    am = torch.full((T,), -1, dtype=torch.int32, device=dev())
    lg = torch.empty((T, Wq.shape[0]), dtype=torch.float32, device=dev()) if want_logits else None
    moe.fp8_head_run(h, to_dev_u16(x), am, lg)
    torch.cuda.synchronize()
    moe.fp8_head_destroy(h)
    return am.cpu().numpy(), None if lg is None else lg.cpu().numpy()


@pytest.mark.parametrize("V,T,H", [(3000, 4, 2560), (64 * 7 + 5, 1, 2560), (1, 2, 2560), (700, 4, 256),
                                   (130, 3, 1024)])
def test_small_head_matches_oracle(V, T, H):
    Wq, s = _quantised(V, H, seed=13)
    x = synth.tokens(H, 13, T)
    lg_o, bd_o, am_o = oracle.head_logits(Wq, s, x)
    am, lg = _run(Wq, s, x)
    assert (np.abs(lg - lg_o) <= bd_o).all()
    for t in range(T):
        if V == 1 or oracle.argmax_margin_ok(lg_o[t], bd_o[t]):
            assert am[t] == am_o[t]


def test_duplicate_rows_lowest_index_wins():
    V, H = 500, 2560
    Wq, s = _quantised(V, H, seed=9)
    x = synth.tokens(H, 9, 1)
    _, _, am_o = oracle.head_logits(Wq, s, x, want_logits=False, want_bounds=False)
    r = int(am_o[0])
    Wq[V - 1], s[V - 1] = Wq[r], s[r]
    Wq[r - 1 if r > 0 else 1], s[r - 1 if r > 0 else 1] = Wq[r], s[r]
    am, _ = _run(Wq, s, x, want_logits=False)
    assert am[0] == min(r - 1 if r > 0 else 1, r)


@pytest.mark.parametrize("T", [1, 4])
def test_full_head_argmax(T):
    m = MANIFEST["head"]
    V, H = m["vocab"], m["hidden"]
    Wq, s = _quantised(V, H, m["seed"])
    x = synth.tokens(H, m["seed"], 4, m["x_attempt"])[:T]
    am, lg = _run(Wq, s, x)
    assert am.tolist() == m["argmax"][:T]
    # sampled rows against the oracle's fp64 logits and fp32 bounds
    rows = np.unique(np.concatenate([np.arange(0, V, 997), np.array(m["argmax"][:T]), [V - 1]]))
    lg_o, bd_o, _ = oracle.head_logits(Wq[rows], s[rows], x)
    assert (np.abs(lg[:, rows] - lg_o) <= bd_o).all()
