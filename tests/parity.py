"""Shared helpers for the GPU parity tests: run the library, run the oracle on
the same generated inputs, compare."""
import numpy as np
import torch

import oracle.rea_oracle as O
import synth
import top_kv_cache_amd as rea
from synth import torch_io

# output tolerance (max-abs) by input dtype
TOL = {"bf16": 2e-2, "f32": 1e-5}


def log(*a):
    print(*a, flush=True)


def device_inputs(w, layer=0, q=None, K=None, V=None):
    q = torch_io.q_device(w, layer) if q is None else q
    K = torch_io.kv_device(w, layer, "k") if K is None else K
    V = torch_io.kv_device(w, layer, "v") if V is None else V
    return q, K, V


def run_library(w, q, K, V, components=True):
    """All four entry points on the device; results copied to host numpy."""
    st = rea.Step(q, K, V, w.G, w.S, w.topk, w.L, w.block_q, rope_theta=w.rope_theta,
                  per_q_head=w.per_q_head, token_segments=w.token_segments)
    res = {"sizes": st.sizes}
    if components:
        sel, nsel, sc = st.score_select(span_scores=True)
        k_win, v_win, q_rot, W = st.gather_rope(sel, nsel)
        out = st.window_attend(q_rot, k_win, v_win, W)
        res.update(sel=sel, nsel=nsel, sc=sc, k_win=k_win, v_win=v_win, q_rot=q_rot, W=W,
                   out=out)
    Hs, nb = st.sizes.n_sel_heads, st.sizes.n_blocks
    assert Hs == w.H_sel
    cap = w.sel_cap
    sel2 = torch.full((nb, Hs, max(cap, 1)), -7, dtype=torch.int32, device=q.device)
    nsel2 = torch.empty((nb, Hs), dtype=torch.int32, device=q.device)
    res["out_step"] = st.decode_step(sel=sel2 if cap > 0 else None, nsel=nsel2)
    res["sel_step"], res["nsel_step"] = sel2[:, :, :cap], nsel2
    torch.cuda.synchronize()
    host = {}
    for k, v in res.items():
        if isinstance(v, torch.Tensor):
            if v.dtype == torch.bfloat16:
                v = v.view(torch.int16).cpu().numpy().view(np.uint16)
                v = synth.bf16_bits_to_f32(v)
            else:
                v = v.cpu().numpy()
        host[k] = v
    return host


def oracle_head(w, layer, h, q64=None, K_h=None, V_h=None):
    """Oracle steps for selection head h alone (KV heads are independent): KV
    head h with its query group, or, when each query head selects, query head h
    within its KV head's group (the oracle runs the whole group, per head)."""
    g = w.g
    hp = h // g if w.per_q_head else h          # KV head
    if q64 is None:
        q64 = synth.to_f32(w.q(layer), w.dtype).astype(np.float64)
    qh = q64[:, hp * g:(hp + 1) * g]
    if K_h is None:
        K_h = synth.to_f32(w.kv(layer, "k", hp, hp + 1), w.dtype).astype(np.float64)
    if V_h is None:
        V_h = synth.to_f32(w.kv(layer, "v", hp, hp + 1), w.dtype).astype(np.float64)
    sel, sc = O.score_select(qh, K_h, w.G, w.S, w.topk, w.L, w.block_q, return_scores=True,
                             per_q_head=w.per_q_head, token_segments=w.token_segments)
    Kw, Vw, qr, W, qpos = O.gather_rope(qh, K_h, V_h, sel, w.G, w.S, w.L, w.block_q,
                                        w.rope_theta, per_q_head=w.per_q_head,
                                        token_segments=w.token_segments)
    out = O.window_attend(qr, Kw, Vw, qpos, w.block_q)
    u = h - hp * g if w.per_q_head else 0       # unit within the group's result
    cols = slice(u, u + 1) if w.per_q_head else slice(0, g)
    res = dict(sel=[s[u] for s in sel], sc=sc[:, u], Kw=[k[u] for k in Kw],
               Vw=[v[u] for v in Vw], q_rot=qr[:, cols], W=W[:, u], out=out[:, cols])
    if mfma_path(w):
        lo, hi = w.mid
        res["eps"] = mfma_span_bounds(qh[:, cols], K_h[0], lo, hi, w.S, w.block_q)
    elif heads_mfma_path(w):
        lo, hi = w.mid
        res["eps"] = heads_span_bounds(qh[0, u], K_h[0], lo, hi, w.S)
    return res


def mfma_path(w):
    """Blocks of 64 bf16 queries with d 128 are scored on MFMA: their span scores
    are approximations within a proven bound (selection stays exact)."""
    return (w.dtype == "bf16" and w.d == 128 and w.block_q == 64 and w.S % 32 == 0
            and w.n_spans > 0 and not w.token_segments)


def heads_mfma_path(w):
    """A decode step with one selection per query head (bf16, d 128, S a
    multiple of 32, one sequence) scores the query heads of a KV head together
    on MFMA: approximate span scores within a proven bound, exact selection."""
    return (w.dtype == "bf16" and w.d == 128 and w.block_q == 1 and w.n_q == 1 and w.per_q_head
            and 2 <= w.g <= 32 and w.S % 32 == 0 and w.n_spans > 0 and not w.token_segments)


GAMMA_HEADS = 128 * 2.0 ** -23


def heads_span_bounds(q_head, K_h, mid_lo, mid_hi, S):
    """Per-span bounds eps[0][j] of the per-query-head MFMA scores, from the
    bound the scoring path states: q_h is bf16, every product with a bf16 key
    is exact in fp32, and the fp32 sum of a token's 128 products is within
    128 * 2^-23 * ||q_h|| * ||k_t|| of the exact score; a span maximum moves by
    at most that with the span's largest key norm.  q_head [d] fp64."""
    e = GAMMA_HEADS * float(np.linalg.norm(q_head))
    kn = np.linalg.norm(K_h[mid_lo:mid_hi], axis=1)
    n_spans = -(-(mid_hi - mid_lo) // S)
    kn = np.concatenate([kn, np.zeros(n_spans * S - kn.size)])
    return e * kn.reshape(n_spans, S).max(axis=1)[None, :]


GAMMA_MFMA = 255 * 2.0 ** -23 * (1 + 1e-6)


def mfma_span_bounds(q_grp, K_h, mid_lo, mid_hi, S, block_q):
    """Per-span error bounds eps[b][j] of the MFMA block scores, from the
    bound the scoring path states: each query's group sum q_eff (fp64) is
    split as hi = bf16(fp32(q_eff)), lo = bf16(fp32(q_eff - hi)); a token score
    summed in fp32 over the 2d exact products of [hi|lo] with a bf16 key is
    within e_i * ||k_t|| of the exact one, with
    e_i = 255 * 2^-23 * (1 + 1e-6) * ||(|hi| + |lo|)|| + ||q_eff - hi - lo||;
    so the span score of a block is within eps_j = (sum_i e_i) * max_{t in j} ||k_t||.

    q_grp [n_q][g][d] fp64 (one selection unit's query heads), K_h [T][d] fp64.
    """
    def bf16(x):
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)
    qe = q_grp.sum(axis=1)                               # exact for bf16 heads
    hi = bf16(qe)
    lo = bf16(qe - hi)
    e = GAMMA_MFMA * np.linalg.norm(np.abs(hi) + np.abs(lo), axis=1) + \
        np.linalg.norm(qe - hi - lo, axis=1)
    E = e.reshape(-1, block_q).sum(axis=1)               # [n_blk]
    kn = np.linalg.norm(K_h[mid_lo:mid_hi], axis=1)
    n_spans = -(-(mid_hi - mid_lo) // S)
    pad = np.full(n_spans * S - kn.size, 0.0)
    kbar = np.concatenate([kn, pad]).reshape(n_spans, S).max(axis=1)
    return E[:, None] * kbar[None, :]


def fused_path(w):
    """rea_decode_step runs steps 2-4 fused, reading the window straight from
    the cache: up to 8 query rows per (block, selection head) on the VALU;
    bf16 d 128 beyond that on MFMA (2-wave workgroups up to 64 rows, 8-wave
    ones with at most 4096 selection entries beyond)."""
    rows = w.block_q * w.g_sel
    mfma_cache = w.dtype == "bf16" and w.d == 128 and rows > 8 and (rows <= 64 or w.sel_cap <= 4096)
    return rows <= 8 or mfma_cache


def compare_head(w, gpu, ora, h, check_windows=True):
    """Assert parity of selection head h; returns the max-abs output error."""
    g, nb = w.g_sel, len(ora["sel"])
    for b in range(nb):
        exp = ora["sel"][b]
        ns = int(gpu["nsel"][b, h])
        got = gpu["sel"][b, h, :ns].tolist() if w.topk > 0 else []
        assert ns == len(exp), (b, h, ns, len(exp))
        assert got == exp, (b, h, sorted(set(got) ^ set(exp))[:10])
        if w.sel_cap > ns:
            assert np.all(gpu["sel"][b, h, ns:] == -1)
        got_step = gpu["sel_step"][b, h, :ns].tolist() if w.topk > 0 else []
        assert got_step == exp and int(gpu["nsel_step"][b, h]) == ns
    if ora["sc"].size:
        ref = ora["sc"]
        diff = np.abs(gpu["sc"][:, h, :] - ref)
        if mfma_path(w) or heads_mfma_path(w):
            # MFMA approximations: every span within its own bound eps_j, the
            # bound the certification of the selection rests on
            eps = ora["eps"]
            worst = float(np.max(np.where(diff > 0, diff / np.maximum(eps, 1e-300), 0.0)))
            assert np.all(diff <= eps), ("span scores beyond eps_j", h, worst)
            ora["eps_used"] = worst
        else:
            scale = max(1.0, float(np.abs(ref).max()))
            assert diff.max() <= 1e-12 * scale, ("span scores", h, float(diff.max()))
    assert np.array_equal(gpu["W"][:, h], ora["W"]), (gpu["W"][:, h], ora["W"])
    if check_windows:
        for b in range(nb):
            Wb = int(ora["W"][b])
            kref = ora["Kw"][b]
            kgot = gpu["k_win"][b, h, :Wb].astype(np.float64)
            slack = 1e-13 * float(np.abs(kref).max()) if kref.size else 0.0
            assert np.all(np.abs(kgot - kref) <= 1.2e-7 * np.abs(kref) + slack), ("k_win", b, h)
            assert np.array_equal(gpu["v_win"][b, h, :Wb].astype(np.float64), ora["Vw"][b]), \
                ("v_win", b, h)
        qref = ora["q_rot"]
        qgot = gpu["q_rot"][:, h * g:(h + 1) * g].astype(np.float64)
        slack = 1e-13 * float(np.abs(qref).max())
        assert np.all(np.abs(qgot - qref) <= 1.2e-7 * np.abs(qref) + slack), ("q_rot", h)
    oref = ora["out"]
    ogot = gpu["out_step"][:, h * g:(h + 1) * g].astype(np.float64)
    err = float(np.abs(ogot - oref).max())
    assert err <= TOL[w.dtype], ("out", h, err)
    if "out" in gpu:
        got = gpu["out"][:, h * g:(h + 1) * g]
        if fused_path(w):
            # rea_decode_step attends straight from the cache: same tolerance,
            # different rounding than window_attend over the written window
            err_sep = float(np.abs(got.astype(np.float64) - oref).max())
            assert err_sep <= TOL[w.dtype], ("out (window_attend)", h, err_sep)
        else:
            assert np.array_equal(got, gpu["out_step"][:, h * g:(h + 1) * g])
    return err
