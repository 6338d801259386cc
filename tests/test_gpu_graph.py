"""rea_decode_step and rea_decode_step_noalloc captured into a HIP graph (the
decode step issues only kernel launches on the caller's stream: no memset,
copy, allocation or host synchronisation), replayed several times with new
query values written into the captured input between replays and eager work
and synchronisations in between; every replay must give the selection and
the output bits that an eager call on the same inputs gives."""
import dataclasses

import pytest
import torch

import synth
import top_kv_cache_amd as rea
from synth import torch_io
from tests.parity import log

pytestmark = pytest.mark.gpu

W = synth.small(name="graph-8b-20k", seed=61, Hq=32, Hkv=8, d=128, T=20000, S=32, topk=40,
                L=1024, needles=2, kv_scaled=True)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_step_replayed_from_a_graph(noalloc):
    dev = torch.device("cuda:0")
    q = torch_io.q_device(W, 0, dev)
    K = torch_io.kv_device(W, 0, "k", device=dev)
    V = torch_io.kv_device(W, 0, "v", device=dev)
    st = rea.Step(q, K, V, W.G, W.S, W.topk, W.L, 1, rope_theta=W.rope_theta)
    ws = st.workspace()
    out = torch.empty((1, W.Hq, W.d), dtype=torch.float32, device=dev)
    sel = torch.empty((1, W.Hkv, W.topk), dtype=torch.int32, device=dev)
    nsel = torch.empty((1, W.Hkv), dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()

    def step(o, sl, ns, w_s, stream):
        if noalloc:
            return st.decode_step_noalloc(out=o, sel=sl, nsel=ns, stream=stream)
        return st.decode_step(out=o, sel=sl, nsel=ns, ws=w_s, stream=stream)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(out, sel, nsel, ws, s)             # warm-up before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(out, sel, nsel, ws, s)
    torch.cuda.synchronize()

    ws_e = st.workspace()
    outs = []
    for i in range(3):
        # new query values in the tensor the graph reads
        wi = dataclasses.replace(W, seed=W.seed + 100 + i)
        q.copy_(torch_io.q_device(wi, 0, dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), sel.clone(), nsel.clone())
        outs.append(got[0])
        # eager work between the replays: the same step on another workspace
        # (the no-allocation variant shares its one scratch array with the graph)
        o_e = torch.empty_like(out)
        s_e = torch.empty_like(sel)
        n_e = torch.empty_like(nsel)
        if noalloc:
            st.decode_step_noalloc(out=o_e, sel=s_e, nsel=n_e)
        else:
            st.decode_step(out=o_e, sel=s_e, nsel=n_e, ws=ws_e)
        torch.cuda.synchronize()
        log(f"[graph] replay {i} (noalloc={noalloc}): max |out| {got[0].abs().max().item():.3f}")
        assert torch.equal(got[2], n_e)
        for h in range(W.Hkv):
            k = int(n_e[0, h])
            assert torch.equal(got[1][0, h, :k], s_e[0, h, :k]), (i, h)
        assert torch.equal(got[0], o_e), (i, float((got[0] - o_e).abs().max()))
    # the replays read the query written before each: their outputs differ
    assert not torch.equal(outs[0], outs[1]) and not torch.equal(outs[1], outs[2])
