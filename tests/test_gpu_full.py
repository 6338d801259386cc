"""Full-size GPU parity on the evaluation workloads.

  * 3B-shaped decode at 4,194,304 tokens: every KV head checked against the
    oracle (selection exact, span scores, window rows, output).
  * 8B-shaped token-level decode at 1,048,576 tokens (3840 single tokens
    selected per KV head): every KV head checked the same way; and the
    per-query-head and token-segment selections at the same size.
  * 8B-shaped chunked prefill (4096 queries appended at 131072, blocks of 64):
    every (block, KV head) selection and every output checked; and one
    512-query chunk at 140,000 tokens (more than 4,096 spans per block).
  * 8B-shaped batched decode of 32 sequences at 32K tokens (equal and ragged
    lengths) as the batched bench builds it: every sequence checked.
  * 8B-shaped decode at 1,048,576 tokens with all 32 layers resident, run
    exactly as bench.py runs it (one shared workspace, rea_decode_step per
    layer): two layers checked in full against the oracle, every layer checked
    for its planted needle spans, selection size and output finiteness.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle.rea_oracle as O
import synth
import top_kv_cache_amd as rea
from synth import torch_io
from tests.parity import TOL, compare_head, device_inputs, log, oracle_head, run_library

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _one_layer(cfg, w=None, needles=True):
    w = synth.config(cfg) if w is None else w
    log(f"[config {cfg}] {w.name}: generating + uploading")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    del K, V
    torch.cuda.empty_cache()
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    errs = []
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64)
        errs.append(compare_head(w, gpu, ora, h))
        if needles:
            planted = [j for (hh, j) in w.needle_spans(0) if hh == h]
            for b in range(len(ora["sel"])):
                assert set(planted) <= set(ora["sel"][b])
        log(f"  head {h}: parity ok, out err {errs[-1]:.2e}")
    log(f"  max-abs out err {max(errs):.3e} (tolerance {TOL[w.dtype]})")


@pytest.mark.timeout(900)
def test_decode_4m_llama3b():
    _one_layer(5)


@pytest.mark.timeout(900)
def test_prefill_chunk_llama8b():
    _one_layer(4)


@pytest.mark.timeout(900)
def test_decode_1m_token_level():
    """Token-level selection at 1,048,576 tokens as the token-level bench runs
    it (spans of one token, the 3840 best: the top-k's large path over 32,640
    group maxima held in registers), one layer of the 8B shape, every KV head
    checked against the oracle: selection exact, token scores, window rows,
    output."""
    w = dataclasses.replace(synth.config(3), S=1, topk=3840)
    w.name = f"{w.name}-token-level"
    _one_layer(3, w, needles=False)


VARIANTS_1M = {
    "per_q_head": dict(per_q_head=True),
    "token_segments": dict(token_segments=True),
    "pages_k127": dict(topk=127),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", list(VARIANTS_1M))
def test_decode_1m_selection_variants(variant):
    """The other selection variants the bench runs at 1,048,576 tokens (8B
    shape, one layer): one selection per query head (8 of the 32 selection
    heads checked, one per KV head at every position in its group), the 120
    best tokens each widened to 32, and the pages' LLaMA3-8B-8K selection of
    127 spans (window exactly 8192; every KV head checked)."""
    w = dataclasses.replace(synth.config(3), **VARIANTS_1M[variant])
    w.name = f"{w.name}-{variant.replace('_', '-')}"
    log(f"[variant] {w.name}: generating + uploading")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    del K, V
    torch.cuda.empty_cache()
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    heads = [u * w.g + u % w.g for u in range(w.Hkv)] if w.per_q_head else list(range(w.H_sel))
    errs = []
    for h in heads:
        ora = oracle_head(w, 0, h, q64)
        errs.append(compare_head(w, gpu, ora, h))
        log(f"  selection head {h}: parity ok, out err {errs[-1]:.2e}")
    log(f"  max-abs out err {max(errs):.3e} (tolerance {TOL[w.dtype]})")


@pytest.mark.timeout(900)
def test_prefill_chunk512_past_4096_spans():
    """A 512-token prefill chunk (8 blocks of 64) at 140,000 tokens with the
    pages' 8B setting (G 32, S 32, 127 spans, L 4096): 4,246 spans per block
    and KV head, more than the 4,096 the MFMA block path's certification
    holds on chip; every (block, KV head) selection and output checked."""
    w = synth.small(name="llama8b-bf16-prefill-chunk512-at-140k", seed=240715184, Hq=32,
                    Hkv=8, d=128, T=140000, n_q=512, block_q=64, G=32, S=32, topk=127,
                    L=4096, needles=8, kv_scaled=True)
    assert w.n_spans > 4096
    log(f"[prefill chunk] {w.name}: {w.n_spans} spans per (block, KV head)")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    del K, V
    torch.cuda.empty_cache()
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    errs = []
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64)
        errs.append(compare_head(w, gpu, ora, h))
        log(f"  head {h}: parity ok, out err {errs[-1]:.2e}")
    log(f"  max-abs out err {max(errs):.3e} (tolerance {TOL[w.dtype]})")


@pytest.mark.timeout(900)
def test_prefill_block_at_1m_tokens():
    """One 64-query block of the 8B shape at 1,048,576 tokens: 32,639 spans per
    KV head scored on MFMA, the certification ranking only its candidate
    spans; selection, span-score bounds and outputs of KV heads 0 and 7
    checked against the oracle."""
    w = synth.small(name="llama8b-bf16-prefill-block-at-1m", seed=240715185, Hq=32, Hkv=8,
                    d=128, T=1048576, n_q=64, block_q=64, G=32, S=32, topk=120, L=4096,
                    needles=8, kv_scaled=True)
    assert w.n_spans == 32639
    log(f"[prefill block] {w.name}: {w.n_spans} spans per KV head")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    del K, V
    torch.cuda.empty_cache()
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    for h in (0, w.Hkv - 1):
        ora = oracle_head(w, 0, h, q64)
        err = compare_head(w, gpu, ora, h)
        log(f"  head {h}: selection exact, worst |s_hat - s| / eps_j {ora['eps_used']:.3g}, "
            f"out err {err:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ragged", [False, True])
def test_decode_batch_32x32k_as_benchmarked(ragged):
    """The batched decode as `bench.py --batch 32 --context 32768 [--ragged]`
    builds it (8B shape, sequence b seeded seed + 1000 b; ragged lengths spread
    over [16384, 32768]), one layer, one rea_decode_batch: every sequence's
    selection compared bit-exactly with the oracle run on that sequence alone,
    and its output within tolerance."""
    B, T = 32, 32768
    base = synth.small(name="llama8b-bf16-decode-batch32-32k", seed=240715190, dtype="bf16",
                       Hq=32, Hkv=8, d=128, T=T, n_q=1, block_q=1, G=32, S=32, topk=120,
                       L=4096, needles=4, kv_scaled=True, layers=1)
    lens = [T - (i * (T // 2)) // (B - 1) for i in range(B)] if ragged else [T] * B
    dev = torch.device("cuda:0")
    q = torch.empty((B, base.Hq, base.d), dtype=torch.bfloat16, device=dev)
    K = torch.empty((B, base.Hkv, T, base.d), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    seqs = [dataclasses.replace(base, seed=base.seed + 1000 * b) for b in range(B)]
    for b, wb in enumerate(seqs):
        q[b] = torch_io.q_device(wb, 0, dev)[0]
        torch_io.kv_device(wb, 0, "k", out=K[b], device=dev)
        torch_io.kv_device(wb, 0, "v", out=V[b], device=dev)
    lengths = torch.tensor(lens, dtype=torch.int64, device=dev)
    db = rea.DecodeBatch(q, K, V, lengths, base.G, base.S, base.topk, base.L,
                         rope_theta=base.rope_theta)
    sel = torch.full((B, base.Hkv, base.topk), -7, dtype=torch.int32, device=dev)
    nsel = torch.empty((B, base.Hkv), dtype=torch.int32, device=dev)
    log(f"[batch] 32 x 32K ({'ragged' if ragged else 'equal'} lengths {lens[-1]}..{lens[0]})")
    out = db.run(sel=sel, nsel=nsel)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    sel_h, nsel_h = sel.cpu().numpy(), nsel.cpu().numpy()

    def f64(t):                         # the device's bf16 values, exactly
        return t.float().cpu().numpy().astype(np.float64)

    err = 0.0
    for b in range(B):
        Tb = lens[b]
        qb, Kb, Vb = f64(q[b:b + 1]), f64(K[b, :, :Tb]), f64(V[b, :, :Tb])
        ref, rsel = O.step(qb, Kb, Vb, base.G, base.S, base.topk, base.L, 1, base.rope_theta)
        for u in range(base.Hkv):
            ns = int(nsel_h[b, u])
            assert ns == len(rsel[0][u]), (b, u, ns)
            assert sel_h[b, u, :ns].tolist() == rsel[0][u], (b, u)
        e = float(np.abs(got[b] - ref[0]).max())
        err = max(err, e)
        assert e <= TOL["bf16"], (b, Tb, e)
    log(f"  32 sequences: selections exact, max-abs out err {err:.3e} (tolerance {TOL['bf16']})")


@pytest.mark.timeout(1100)
def test_decode_1m_32_layers_as_benchmarked():
    w = synth.config(3)
    dev = torch.device("cuda:0")
    steps, outs, sels, nsels = [], [], [], []
    for layer in range(w.n_layers):
        q = torch_io.q_device(w, layer, dev)
        K = torch_io.kv_device(w, layer, "k", device=dev)
        V = torch_io.kv_device(w, layer, "v", device=dev)
        steps.append(rea.Step(q, K, V, w.G, w.S, w.topk, w.L, w.block_q, rope_theta=w.rope_theta))
        outs.append(torch.empty((1, w.Hq, w.d), dtype=torch.float32, device=dev))
        sels.append(torch.empty((1, w.Hkv, w.topk), dtype=torch.int32, device=dev))
        nsels.append(torch.empty((1, w.Hkv), dtype=torch.int32, device=dev))
        if layer % 8 == 7:
            log(f"  uploaded {layer + 1}/{w.n_layers} layers")
    ws = steps[0].workspace()
    for rep in range(2):                     # the second pass reuses a dirty workspace
        for li, st in enumerate(steps):
            st.decode_step(out=outs[li], sel=sels[li], nsel=nsels[li], ws=ws)
        torch.cuda.synchronize()
    sel = [s.cpu().numpy() for s in sels]
    nsel = [n.cpu().numpy() for n in nsels]
    out = [o.cpu().numpy() for o in outs]
    for layer in range(w.n_layers):
        assert np.all(nsel[layer] == w.topk)
        assert np.all(np.isfinite(out[layer]))
        for (h, j) in w.needle_spans(layer):
            assert j in sel[layer][0, h], (layer, h, j)
    del steps
    torch.cuda.empty_cache()
    for layer in (0, w.n_layers - 1):
        q64 = synth.to_f32(w.q(layer), w.dtype).astype(np.float64)
        for h in range(w.Hkv):
            ora = oracle_head(w, layer, h, q64)
            assert sel[layer][0, h].tolist() == ora["sel"][0], (layer, h)
            err = float(np.abs(out[layer][:, h * w.g:(h + 1) * w.g] - ora["out"]).max())
            assert err <= TOL[w.dtype], (layer, h, err)
            log(f"  layer {layer} head {h}: selection exact, out err {err:.2e}")
