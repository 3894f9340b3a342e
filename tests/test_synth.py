"""Generator tests (CPU): published SplitMix64 vector, determinism, chunking, distributions."""
import numpy as np

import synth


def test_splitmix64_published_vector():
    # First outputs of SplitMix64 (Steele, Lea & Flood 2014) seeded with 1234567, as listed by the
    # reference C implementation's test vector.  sm(s, i) is the (i+1)-th output.
    L = synth.host_lib()
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
            16408922859458223821]
    assert [L.synth_hash(1234567, i) for i in range(5)] == want


def test_chunks_equal_whole():
    k = synth.key(3, 7, synth.TENSOR_W13, 11, 0)
    whole = synth.codes(1000, k)
    assert (np.concatenate([synth.codes(333, k), synth.codes(667, k, i0=333)]) == whole).all()
    ks = synth.key(3, 7, synth.TENSOR_W13S, 11, 0)
    assert (np.concatenate([synth.scales(10, ks), synth.scales(90, ks, i0=10)]) == synth.scales(100, ks)).all()
    kn = synth.key(3, 0, synth.TENSOR_HEAD, 0, 0)
    assert (np.concatenate([synth.normal_f32(5, kn, 0.02), synth.normal_f32(7, kn, 0.02, i0=5)])
            == synth.normal_f32(12, kn, 0.02)).all()


def test_keys_separate_coordinates():
    base = synth.key(1, 0, 1, 0, 0)
    others = {synth.key(2, 0, 1, 0, 0), synth.key(1, 1, 1, 0, 0), synth.key(1, 0, 2, 0, 0),
              synth.key(1, 0, 1, 1, 0), synth.key(1, 0, 1, 0, 1)}
    assert base not in others and len(others) == 5


def test_distributions():
    k = synth.key(0, 0, synth.TENSOR_W13, 0, 0)
    c = synth.codes(1 << 20, k)
    nib = np.concatenate([c & 0xF, c >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.95 * counts.mean() and counts.max() < 1.05 * counts.mean()
    s = synth.scales(1 << 16, synth.key(0, 0, synth.TENSOR_W13S, 0, 0))
    assert set(np.unique(s)) == {121, 122, 123, 124, 125}
    r = synth.router(synth.FLASH, 0).astype(np.uint32)
    v = (r << 16).view(np.float32)
    assert abs(v.std() - 0.02) < 0.0005 and abs(v.mean()) < 0.0005
    x = synth.tokens(2560, 0, 4)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xv.std() - 1.0) < 0.05
    w = synth.head_weights(1000, 2560, seed=4, rows=100)
    assert abs(w.std() - 0.02) < 0.001


def test_expert_shapes():
    t = synth.expert(synth.FLASH, 1, 0, 512)
    assert t["w13"].shape == (1536, 1280) and t["w13_s"].shape == (1536, 80)
    assert t["w2"].shape == (2560, 384) and t["w2_s"].shape == (2560, 24)
    per_expert = sum(v.nbytes for v in t.values())
    assert per_expert == 3_133_440


def test_tokens_correlated_mix_and_rounding():
    """Correlated verify tokens: token 0 is bit-equal to tokens()'s token 0 (the same normal draw and
    the same round-to-nearest-even bf16 rounding, done here in numpy and in C there); token t >= 1 has
    correlation rho with token 0 and rho^2 with the other mixed tokens."""
    H, rho = 2560, 0.9
    x = synth.tokens_correlated(H, 5, 3, rho, 0)
    assert x.shape == (3, H) and x.dtype == np.uint16
    assert (x[0] == synth.tokens(H, 5, 1, 0)[0]).all()
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    c = np.corrcoef(f)
    assert abs(c[0, 1] - rho) < 0.02 and abs(c[0, 2] - rho) < 0.02
    assert abs(c[1, 2] - rho * rho) < 0.03
    assert (synth.tokens_correlated(H, 5, 3, rho, 0) == x).all()
