"""GPU parity of the chunked prefill (rea_prefill) against the oracle run chunk
by chunk on the same cut caches: each chunk's queries see the cache up to the
end of their chunk and are selected in blocks as the plan states."""
import numpy as np
import pytest
import torch

import oracle.rea_oracle as O
import synth
import top_kv_cache_amd as rea
from synth import torch_io
from tests.parity import TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


CASES = {
    # bf16 d 128 blocks of 64: MFMA scoring + certification and MFMA attention
    # from the cache; the last chunk (56 tokens) takes blocks of 56 on the VALU
    # scoring path
    "bf16_mfma": dict(Hq=8, Hkv=2, d=128, T=3000, S=16, topk=12, G=8, L=256, needles=0,
                      block_q=64, chunk=128),
    # fp32 d 64 blocks of 16 on the VALU paths
    "f32_valu": dict(dtype="f32", Hq=4, Hkv=2, d=64, T=700, S=8, topk=6, G=4, L=64, needles=0,
                     block_q=16, chunk=32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle_chunk_by_chunk(name):
    kw = dict(CASES[name])
    bq, chunk = kw.pop("block_q"), kw.pop("chunk")
    w = synth.small(n_q=kw["T"], block_q=1, **kw)
    q = torch_io.q_device(w)                    # every prompt token is a query
    K, V = torch_io.kv_device(w, 0, "k"), torch_io.kv_device(w, 0, "v")
    pf = rea.Prefill(q, K, V, w.G, w.S, w.topk, w.L, bq, chunk, rope_theta=w.rope_theta)
    log(f"[prefill] {name}: T={w.T}, {len(pf.plan)} chunks, first {pf.plan[0]}, last {pf.plan[-1]}")
    out = pf.run()
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    g, err = w.g, 0.0
    for h in range(w.Hkv):
        K_h = synth.to_f32(w.kv(0, "k", h, h + 1), w.dtype).astype(np.float64)[0]
        V_h = synth.to_f32(w.kv(0, "v", h, h + 1), w.dtype).astype(np.float64)[0]
        for start, n, b in pf.plan:
            end = start + n
            ref, _ = O.step(q64[start:end, h * g:(h + 1) * g], K_h[None, :end], V_h[None, :end],
                            w.G, w.S, w.topk, w.L, b, w.rope_theta)
            e = float(np.abs(got[start:end, h * g:(h + 1) * g] - ref).max())
            err = max(err, e)
            assert e <= TOL[w.dtype], (name, h, start, n, b, e)
    log(f"  max-abs out err {err:.3e} (tolerance {TOL[w.dtype]})")
