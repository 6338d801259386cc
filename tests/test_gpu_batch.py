"""GPU parity of the batched decode (rea_decode_batch) against the oracle run
on each sequence alone: ragged lengths (from a single token to the capacity),
cache rows past a sequence's length filled with large values that would be
selected if they were read, both selection granularities, token-level spans,
and an 8B-shaped batch at 32K tokens."""
import dataclasses

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
    "bf16_d128_ragged": (dict(Hq=8, Hkv=2, d=128, T=3000, S=16, topk=12, G=4, L=64),
                         [3000, 1, 700, 2047, 129, 68]),
    "bf16_d128_ragged_per_q_head": (dict(Hq=8, Hkv=2, d=128, T=3000, S=16, topk=12, G=4, L=64,
                                         per_q_head=True), [2999, 5, 1800, 640]),
    "f32_d64_token_level": (dict(dtype="f32", Hq=4, Hkv=2, d=64, T=1500, S=1, topk=40, G=4,
                                 L=32), [1500, 300, 37, 1100]),
    "bf16_d64_g3_partial_spans": (dict(Hq=6, Hkv=2, d=64, T=2000, S=20, topk=9, G=2, L=50),
                                  [2000, 1999, 1013, 77, 52]),
    "bf16_d128_token_segments": (dict(Hq=8, Hkv=2, d=128, T=2500, S=16, topk=10, G=4, L=64,
                                      token_segments=True), [2500, 2, 900, 1777]),
    "bf16_g16_mfma_attention": (dict(Hq=32, Hkv=2, d=128, T=2200, S=32, topk=10, G=4, L=128),
                                [2200, 700, 1500]),
    "llama8b_32k": (dict(Hq=32, Hkv=8, d=128, T=32768, S=32, topk=120, G=32, L=4096,
                         needles=4, kv_scaled=True), [32768, 30000, 24577, 8300]),
}


def _bits_to_f64(t, dtype):
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(
            np.float64)
    return t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_batch_matches_oracle_per_sequence(name):
    kw, lens = CASES[name]
    kw = dict(kw)
    pqh = kw.pop("per_q_head", False)
    tseg = kw.pop("token_segments", False)
    B = len(lens)
    needles = kw.pop("needles", 1)
    base = synth.small(name=name, seed=300, needles=needles, per_q_head=pqh,
                       token_segments=tseg, **kw)
    seqs = [dataclasses.replace(base, seed=300 + b, name=f"{name}-{b}") for b in range(B)]
    dev = torch.device("cuda:0")
    dt = torch_io.torch_dtype(base)
    q = torch.empty((B, base.Hq, base.d), dtype=dt, device=dev)
    K = torch.empty((B, base.Hkv, base.T, base.d), dtype=dt, device=dev)
    V = torch.empty_like(K)
    for b, w in enumerate(seqs):
        q[b] = torch_io.q_device(w, 0, dev)[0]
        torch_io.kv_device(w, 0, "k", out=K[b], device=dev)
        torch_io.kv_device(w, 0, "v", out=V[b], device=dev)
        K[b, :, lens[b]:] = 40.0          # past the sequence: would win any selection
        V[b, :, lens[b]:] = 1000.0
    lengths = torch.tensor(lens, dtype=torch.int64, device=dev)
    db = rea.DecodeBatch(q, K, V, lengths, base.G, base.S, base.topk, base.L,
                         rope_theta=base.rope_theta, per_q_head=pqh, token_segments=tseg)
    Hs = db.sizes.n_sel_heads
    sel = torch.full((B, Hs, max(base.sel_cap, 1)), -7, dtype=torch.int32, device=dev)
    nsel = torch.empty((B, Hs), dtype=torch.int32, device=dev)
    log(f"[batch] {name}: B={B} lengths={lens} H_sel={Hs} ws={db.ws_bytes}")
    out = db.run(sel=sel, nsel=nsel)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    sel_h, nsel_h = sel.cpu().numpy(), nsel.cpu().numpy()
    err = 0.0
    for b in range(B):
        Tb = lens[b]
        qb = _bits_to_f64(q[b:b + 1], base.dtype)
        Kb = _bits_to_f64(K[b, :, :Tb], base.dtype)
        Vb = _bits_to_f64(V[b, :, :Tb], base.dtype)
        ref, rsel = O.step(qb, Kb, Vb, base.G, base.S, base.topk, base.L, 1, base.rope_theta,
                           per_q_head=pqh, token_segments=tseg)
        for u in range(Hs):
            ns = int(nsel_h[b, u])
            assert ns == len(rsel[0][u]), (b, u, ns, len(rsel[0][u]))
            assert sel_h[b, u, :ns].tolist() == rsel[0][u], (b, u)
        e = float(np.abs(got[b] - ref[0]).max())
        err = max(err, e)
        assert e <= TOL[base.dtype], (b, Tb, e)
    log(f"  max-abs out err {err:.3e} (tolerance {TOL[base.dtype]})")


def test_batch_of_one_equals_decode_step():
    """A batch of one sequence at full length runs the same kernels as
    rea_decode_step on that sequence: identical selection and output bits."""
    w = synth.small(Hq=8, Hkv=2, d=128, T=2500, S=32, topk=10, G=4, L=128, needles=2)
    dev = torch.device("cuda:0")
    q = torch_io.q_device(w, 0, dev)
    K = torch_io.kv_device(w, 0, "k", device=dev)
    V = torch_io.kv_device(w, 0, "v", device=dev)
    st = rea.Step(q, K, V, w.G, w.S, w.topk, w.L, 1, rope_theta=w.rope_theta)
    a = st.decode_step()
    db = rea.DecodeBatch(q, K[None], V[None], torch.tensor([w.T], dtype=torch.int64, device=dev),
                         w.G, w.S, w.topk, w.L, rope_theta=w.rope_theta)
    b = db.run()
    torch.cuda.synchronize()
    assert torch.equal(a.view(-1), b.view(-1))
