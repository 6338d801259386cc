"""The seeded generator: C fill == numpy twin bit-for-bit; recipe sanity."""
import numpy as np
import pytest

import synth


def test_splitmix64_first_output():
    # SplitMix64 from state 0: first output of the published generator
    assert synth.sm64(0, 0) == 0xE220A8397B1DCDAF
    assert synth.lib().synth_sm64(0, 0) == 0xE220A8397B1DCDAF
    n = np.arange(1000, dtype=np.uint64)
    a = synth.sm64_np(12345, n)
    b = np.array([synth.sm64(12345, int(i)) for i in n], dtype=np.uint64)
    assert np.array_equal(a, b)


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    # 1.00390625 = 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0078125)
    assert back[3] == -2.5
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)   # half an ulp


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_c_matches_numpy(cfg):
    w = synth.config(cfg)
    rng = np.random.default_rng(cfg)
    assert np.array_equal(w.q(0, impl="c"), w.q(0, impl="np"))
    # random sub-blocks, plus the block holding the first needle
    blocks = []
    for _ in range(3):
        h0 = int(rng.integers(0, w.Hkv))
        t0 = int(rng.integers(0, w.T - 40))
        blocks.append((h0, min(h0 + 2, w.Hkv), t0, t0 + 40))
    nd = w._needle_rows(0)
    if nd:
        h, a = nd[0]
        blocks.append((h, h + 1, a - 3, a + w.S + 3))
    layer = w.n_layers - 1
    for (h0, h1, t0, t1) in blocks:
        for which in "kv":
            a = w.kv(layer, which, h0, h1, t0, t1, impl="c")
            b = w.kv(layer, which, h0, h1, t0, t1, impl="np")
            assert np.array_equal(a, b), (cfg, which, h0, t0)


def test_needles_and_recipe():
    w = synth.config(2)
    nd = w.needle_spans(0)
    assert len(nd) == w.Hkv * w.needles
    for h in range(w.Hkv):
        js = [j for (hh, j) in nd if hh == h]
        assert len(set(js)) == len(js) == w.needles
        assert all(0 <= j < (w.mid[1] - w.mid[0]) // w.S for j in js)
    # a needle span points along the group's query sum
    h, j = nd[0]
    lo = w.mid[0]
    blk = synth.to_f32(w.kv(0, "k", h, h + 1, lo + j * w.S, lo + (j + 1) * w.S), "bf16")[0]
    c = w.needle_centre(0)[h]
    cos = blk @ c / (np.linalg.norm(blk, axis=1) * np.linalg.norm(c))
    assert np.all(cos > 0.95)
    # per-channel scales in [0.5, 2]
    s = w.scale("k", 0)
    assert s.min() >= 0.5 and s.max() <= 2.0
    # Gaussian body
    x = synth.to_f32(w.kv(0, "v", 0, 1, 1000, 3000), "bf16")[0] / w.scale("v", 0)[0]
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_quantile_table():
    assert synth.NQ.dtype == np.float32 and synth.NQ.shape == (65536,)
    assert np.all(np.diff(synth.NQ) > 0)
    assert np.allclose(synth.NQ, -synth.NQ[::-1])
    assert abs(float(synth.NQ.astype(np.float64).std()) - 1) < 1e-3
