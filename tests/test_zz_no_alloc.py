"""rea_decode_step_noalloc (the decode step run on the library's fixed scratch
array) against rea_decode_step with a caller's workspace, through the C ABI:
identical selections and outputs on consecutive calls, each problem smaller
than the one before, so every call after the first finds the scratch array
holding the previous call's data."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import top_kv_cache_amd as rea
from tests.parity import device_inputs, log

pytestmark = pytest.mark.gpu

CALLS = [
    # 8B-shaped decode at 65,536 tokens (scoring, top-k, fused attention)
    synth.small(name="noalloc-8b-64k", seed=41, Hq=32, Hkv=8, d=128, T=65536, S=32, topk=120,
                L=4096, needles=4, kv_scaled=True),
    # a smaller decode with other hyperparameters and a ragged last span
    synth.small(name="noalloc-8b-9000", seed=42, Hq=32, Hkv=8, d=128, T=9000, S=24, topk=40,
                L=1000, needles=2),
    # two blocks of 64 queries: MFMA scoring, certification, MFMA attention
    synth.small(name="noalloc-blocks", seed=43, Hq=8, Hkv=2, d=128, T=3000, n_q=128,
                block_q=64, S=32, topk=12, L=256, needles=0),
]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _run(w, noalloc):
    q, K, V = device_inputs(w)
    st = rea.Step(q, K, V, w.G, w.S, w.topk, w.L, w.block_q, rope_theta=w.rope_theta)
    assert st.sizes.ws_decode_step <= rea.NOALLOC_SCRATCH_BYTES
    nb, Hs = st.sizes.n_blocks, st.sizes.n_sel_heads
    sel = torch.full((nb, Hs, w.topk), -7, dtype=torch.int32, device=q.device)
    nsel = torch.full((nb, Hs), -7, dtype=torch.int32, device=q.device)
    out = torch.full((w.n_q, w.Hq, w.d), float("nan"), dtype=torch.float32, device=q.device)
    if noalloc:
        # through the C ABI directly
        L = rea.lib()
        status = L.rea_decode_step_noalloc(ctypes.byref(st.prob), ctypes.byref(st.par),
                                           ctypes.c_void_p(out.data_ptr()),
                                           ctypes.c_void_p(sel.data_ptr()),
                                           ctypes.c_void_p(nsel.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert status == 0, L.rea_last_error().decode()
    else:
        st.decode_step(out=out, sel=sel, nsel=nsel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy(), nsel.cpu().numpy()


def test_noalloc_matches_decode_step_on_consecutive_calls():
    sizes = []
    for w in CALLS:
        log(f"[noalloc] {w.name}: T={w.T} n_q={w.n_q} block_q={w.block_q} S={w.S} k={w.topk}")
        out_n, sel_n, nsel_n = _run(w, noalloc=True)
        out_r, sel_r, nsel_r = _run(w, noalloc=False)
        assert np.array_equal(nsel_n, nsel_r)
        assert np.array_equal(sel_n, sel_r)
        assert np.all(np.isfinite(out_n))
        assert np.array_equal(out_n, out_r), float(np.abs(out_n - out_r).max())
        sizes.append(w.T * w.Hkv)
    assert sizes == sorted(sizes, reverse=True)
    # and once more on the largest problem, after the smaller ones
    out_n, sel_n, _ = _run(CALLS[0], noalloc=True)
    out_r, sel_r, _ = _run(CALLS[0], noalloc=False)
    assert np.array_equal(sel_n, sel_r) and np.array_equal(out_n, out_r)


def test_noalloc_rejects_problems_beyond_the_scratch_array():
    # token-level selection at 1M tokens needs about 70 MB of scratch
    w = synth.config(3)
    FAKE = 0x10000
    p = rea.problem(FAKE, FAKE, FAKE, dtype=rea.REA_BF16, n_q=1, Hq=w.Hq, Hkv=w.Hkv, d=w.d,
                    T=w.T, stride_head=w.T * w.d, stride_tok=w.d)
    a = rea.params(w.G, 1, 3840, w.L, 1)
    assert rea.query_sizes(p, a).ws_decode_step > rea.NOALLOC_SCRATCH_BYTES
    L = rea.lib()
    st = L.rea_decode_step_noalloc(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, None)
    assert st == rea.STATUS.index("REA_EWORKSPACE")
    assert "scratch" in L.rea_last_error().decode()
