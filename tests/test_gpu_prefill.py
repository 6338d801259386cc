"""GPU parity of the chunked prefill (rea_prefill) against the oracle run chunk
by chunk on the same cut caches: each chunk's queries see the cache up to the
end of their chunk and are selected in blocks as the plan states.  Every
block's selection is compared with the oracle's bit-exactly (rea_prefill
returns the selections of all the plan's blocks), and the outputs within the
stated tolerance."""
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
    # bf16 d 128 blocks of 64, S 32: MFMA scoring + certification and MFMA
    # attention from the cache (one workspace, the RoPE table kept across
    # chunks); the last chunk (56 tokens) takes blocks of 56 on the VALU
    # scoring path
    "bf16_mfma": dict(Hq=8, Hkv=2, d=128, T=3000, S=32, topk=12, G=8, L=256, needles=2,
                      block_q=64, chunk=128),
    # fp32 d 64 blocks of 16 on the VALU paths
    "f32_valu": dict(dtype="f32", Hq=4, Hkv=2, d=64, T=700, S=8, topk=6, G=4, L=64, needles=0,
                     block_q=16, chunk=32),
    # the pages' LLaMA3-8B-8K setting (global 32, span 32, 127 spans, local
    # 4096, chunks of 512; window 8192) in blocks of 64 on the 8B shape; the
    # chunks past 8192 tokens select 127 of up to 319 spans
    "llama8b_pages_k127": dict(Hq=32, Hkv=8, d=128, T=14336, S=32, topk=127, G=32, L=4096,
                               needles=8, kv_scaled=True, block_q=64, chunk=512,
                               out_heads=(0, 5)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle_chunk_by_chunk(name):
    kw = dict(CASES[name])
    bq, chunk = kw.pop("block_q"), kw.pop("chunk")
    out_heads = kw.pop("out_heads", None)
    w = synth.small(name=name, n_q=kw["T"], block_q=1, **kw)
    q = torch_io.q_device(w)                    # every prompt token is a query
    K, V = torch_io.kv_device(w, 0, "k"), torch_io.kv_device(w, 0, "v")
    pf = rea.Prefill(q, K, V, w.G, w.S, w.topk, w.L, bq, chunk, rope_theta=w.rope_theta)
    log(f"[prefill] {name}: T={w.T}, {len(pf.plan)} chunks, {pf.n_blocks} blocks, "
        f"first {pf.plan[0]}, last {pf.plan[-1]}")
    sel_d, nsel_d = pf.selection_buffers()
    sel_d.fill_(-7)
    out = pf.run(sel=sel_d, nsel=nsel_d)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    sel, nsel = sel_d.cpu().numpy(), nsel_d.cpu().numpy()
    del q, K, V, out
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    g, err, n_real = w.g, 0.0, 0
    for h in range(w.Hkv):
        K_h = synth.to_f32(w.kv(0, "k", h, h + 1), w.dtype).astype(np.float64)[0]
        V_h = synth.to_f32(w.kv(0, "v", h, h + 1), w.dtype).astype(np.float64)[0]
        check_out = out_heads is None or h in out_heads
        for (start, n, b), fb in zip(pf.plan, pf.first_block):
            end = start + n
            qc = q64[start:end, h * g:(h + 1) * g]
            ref_sel = O.score_select(qc, K_h[None, :end], w.G, w.S, w.topk, w.L, b)
            for bi in range(n // b):
                exp = ref_sel[bi][0]
                ns = int(nsel[fb + bi, h])
                assert ns == len(exp), (name, h, start, bi, ns, len(exp))
                assert sel[fb + bi, h, :ns].tolist() == exp, \
                    (name, h, start, bi, sorted(set(sel[fb + bi, h, :ns].tolist()) ^ set(exp))[:8])
                assert np.all(sel[fb + bi, h, ns:] == -1), (name, h, start, bi)
                n_spans = O.regions(end, w.G, w.L)
                n_real += 0 < len(exp) < -(-(n_spans[3] - n_spans[2]) // w.S)
            if not check_out:
                continue
            Kw, Vw, qr, _, qpos = O.gather_rope(qc, K_h[None, :end], V_h[None, :end], ref_sel,
                                                w.G, w.S, w.L, b, w.rope_theta)
            ref = O.window_attend(qr, Kw, Vw, qpos, b)
            e = float(np.abs(got[start:end, h * g:(h + 1) * g] - ref).max())
            err = max(err, e)
            assert e <= TOL[w.dtype], (name, h, start, n, b, e)
    log(f"  every block's selection exact ({n_real} (block, head) selections chose among "
        f"more spans than they keep); max-abs out err {err:.3e} (tolerance {TOL[w.dtype]})")
    assert n_real > 0
