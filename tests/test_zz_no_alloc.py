"""The LM head's entry point that allocates nothing (fp8_head_run_noalloc), through the C ABI: on the
caller's row-major weights, its argmax and logits equal those of fp8_head_run on a handle built
from the same weights, bit for bit, on two calls in a row (the second with fewer rows and tokens,
so the shared scratch holds the first call's partials when it starts), and vocabularies beyond its
scratch are refused before any device work."""
import numpy as np
import pytest
import torch

import mxfp4_expert_gemv_amd as moe
import oracle
import synth
from gpu_cases import dev, to_dev_u16

pytestmark = pytest.mark.gpu


def _case(V, H, T, seed):
    W = synth.head_weights(V, H, seed, rows=V)
    Wq, s = oracle.head_quantize(W)
    x = synth.tokens(H, seed, T)
    return torch.from_numpy(Wq).to(dev()), torch.from_numpy(s).to(dev()), to_dev_u16(x)


def _with_handle(w, s, x):
    T, V = x.shape[0], w.shape[0]
    h = moe.fp8_head_create(w, s)
    am = torch.full((T,), -1, dtype=torch.int32, device=dev())
    lg = torch.empty((T, V), dtype=torch.float32, device=dev())
    moe.fp8_head_run(h, x, am, lg)
    torch.cuda.synchronize()
    moe.fp8_head_destroy(h)
    return am.cpu().numpy(), lg.cpu().numpy()


def _no_alloc(w, s, x):
    T, V = x.shape[0], w.shape[0]
    am = torch.full((T,), -1, dtype=torch.int32, device=dev())
    lg = torch.empty((T, V), dtype=torch.float32, device=dev())
    moe.fp8_head_run_noalloc(w, s, x, am, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), lg.cpu().numpy()


def test_no_alloc_head_equals_the_handle_head_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = _case(50000, 2560, 4, 31)     # 50,000 rows of 2,560, 4 tokens
    small = _case(64 * 11 + 5, 1024, 2, 32)  # then fewer rows (a ragged last tile) and 2 tokens
    for w, s, x in (big, small):
        am_h, lg_h = _with_handle(w, s, x)
        am_n, lg_n = _no_alloc(w, s, x)
        assert (am_n == am_h).all(), (am_n, am_h)
        assert (lg_n.view(np.uint32) == lg_h.view(np.uint32)).all()
        # and the argmax is the oracle's where it is well posed
        lg_o, bd_o, am_o = oracle.head_logits(w.cpu().numpy(), s.cpu().numpy(),
                                              x.view(torch.int16).cpu().numpy().view(np.uint16))
        assert (np.abs(lg_n - lg_o) <= bd_o).all()
        for t in range(x.shape[0]):
            if oracle.argmax_margin_ok(lg_o[t], bd_o[t]):
                assert am_n[t] == am_o[t]


def test_no_alloc_head_refuses_vocab_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = torch.zeros((moe.NOALLOC_MAX_VOCAB + 1, 256), dtype=torch.uint8, device=dev())
    s = torch.ones((moe.NOALLOC_MAX_VOCAB + 1,), dtype=torch.float32, device=dev())
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=dev())
    am = torch.empty((1,), dtype=torch.int32, device=dev())
    with pytest.raises(moe.MoeError) as ei:
        moe.fp8_head_run_noalloc(w, s, x, am)
    assert ei.value.status == -1 and "no-allocation limit" in str(ei.value)
