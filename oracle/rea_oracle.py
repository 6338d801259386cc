"""Plain fp64 CPU oracle for the ReAttention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it, and it shares no code, table or constant with the GPU path.

What it computes, for one layer, one batch entry
(q: [n_q][Hq][d] un-rotated queries; K, V: [Hkv][T][d] pre-RoPE cache whose
last n_q rows belong to the queries themselves):

  1. regions   global [0, G'), middle [G', T-L'), local [T-L', T), with
               G' = min(G, T), L' = min(L, T-G')
  2. spans     the middle cut into spans of S tokens from its start; the last
               span may be shorter
  3. scores    s[i,h,t] = sum_g q[i, h*g_sz+g] . K[h,t]  (no RoPE, no scale)
  4. span      sigma_b[h,j] = sum over the block's queries i of
     scores    max over span j's tokens t of s[i,h,t]
  5. top-k     the min(k, n_spans) largest sigma, ties to the lower span
               index, emitted in ascending span order
  6. window    [0, G') ++ selected spans in order ++ [T-L', T); window row w
               gets position w
  7. RoPE      rotate-half rotary embedding at the window positions, for the
               window keys and for the queries (a query sits at the window row
               of its own key)
  8. attention causal softmax attention over the window, scale 1/sqrt(d)

Sources (the page title and the part of it each step follows):
  * "ReAttention: Training-Free Infinite Context with Finite Attention Scope",
    arXiv abstract (mlsanity.com page): position-agnostic top-k attention runs
    before ordinary position-aware self-attention.
  * the same title's research-map summary (atlas.scime.ai), section
    "Approach": middle KV segments are chosen by the dot product of the query
    with un-positioned keys, concatenated with the global and local caches, and
    only then given positional embeddings, so positions stay inside the
    pre-trained range.
  * the same title's OpenReview discussion (paperhub.cn copy):
      - "Decoding Phase" pseudocode: append to the cache first, score the
        middle slice key[G:-L], top-k, concatenate global ++ recalled ++ local
        for both K and V, attend;
      - "Prefilling Phase" pseudocode: the same per chunk (its concat slices
        are garbled; the decoding slices are used);
      - the NIAH reply's hyperparameter list for LLaMA3-8B-8K: global 32,
        span ("seg_size") 32, 127 spans, local 4096, chunk 512;
      - the reply on token eviction: nothing is evicted and selection is
        redone per head, layer and step.

Readings taken where the pages are silent:
  * GQA: one selection per KV head, scoring with the sum of the group's
    query-head logits (step 3).  Variant (per_q_head=True): one selection per
    query head with its own logits, its window gathered from its group's KV
    head.  Token-level selection is the special case S = 1.
  * token segments (token_segments=True): the discussion's InfLLM reply says
    ReAttention selects from the K cache directly rather than from blocks cut
    in advance; read as: the k best tokens, each widened to S tokens centred
    on it, clipped to the middle, overlaps merged.
  * span reduce: max over the span's tokens (step 4); a block of queries sums
    its queries' span maxima.
  * ties: lower span index first (step 5).
  * remainder: a partial last span, scored over and gathered with its real
    length.
  * RoPE: rotate-half pairing (c, c + d/2), inverse frequency
    theta^(-2c/d), positions 0..W-1, angles in fp64.

Arithmetic: products of bf16/fp32 inputs are exact in fp64; sums are fp64.  The
top-k decision is made exact by recomputing, with ``fractions.Fraction``, every
span whose fp64 score lies within 1e-9 * max|sigma| of the k-th one (fp64 error
here is below 1e-12 relative).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

GUARD_REL = 1e-9


# --------------------------------------------------------------------------
# 1-2. regions and spans
# --------------------------------------------------------------------------
def regions(T: int, G: int, L: int):
    """(G', L', mid_lo, mid_hi).  Global [0,G'), middle [G',T-L'), local [T-L',T)."""
    Gp = min(G, T)
    Lp = min(L, T - Gp)
    return Gp, Lp, Gp, T - Lp


def span_list(mid_lo: int, mid_hi: int, S: int):
    """Spans [a, b) tiling the middle from its start; the last may be short."""
    out = []
    a = mid_lo
    while a < mid_hi:
        out.append((a, min(a + S, mid_hi)))
        a += S
    return out


# --------------------------------------------------------------------------
# 3-4. scores
# --------------------------------------------------------------------------
def selection_units(Hq: int, Hkv: int, per_q_head: bool = False):
    """(KV head, query heads) of every independent selection.

    Default: one selection per KV head, scored with the summed logits of the
    query heads of its GQA group.  per_q_head: one selection per query head,
    scored with that head's own logits against its group's KV head (the
    discussion's remark that selection is made for each attention head).
    """
    g = Hq // Hkv
    if per_q_head:
        return [(hq // g, [hq]) for hq in range(Hq)]
    return [(h, list(range(h * g, (h + 1) * g))) for h in range(Hkv)]


def token_scores(q_blk: np.ndarray, K_h: np.ndarray, qheads,
                 mid_lo: int, mid_hi: int) -> np.ndarray:
    """s[i, t - mid_lo] = sum over query heads hq in qheads of q[i, hq] . K_h[t],
    for t in the middle.

    q_blk: [nb][Hq][d] fp64, K_h: [T][d] fp64.  Un-rotated, unscaled.
    """
    nb, _, d = q_blk.shape
    m = len(qheads)
    Qh = q_blk[:, qheads, :].reshape(nb * m, d)                   # [nb*m][d]
    Km = K_h[mid_lo:mid_hi]                                       # [N][d]
    per_head = Qh @ Km.T                                          # [nb*m][N]
    return per_head.reshape(nb, m, -1).sum(axis=1)                # [nb][N]


def span_scores_from_tokens(s: np.ndarray, spans, mid_lo: int) -> np.ndarray:
    """sigma[j] = sum_i max_{t in span j} s[i, t]; -0 canonicalised to +0.

    s: [nb][N] token scores of the block's queries over the middle.  Spans of
    full length S are reduced together through a [nb][n_full][S] view.
    """
    if not spans:
        return np.zeros(0)
    nb = s.shape[0]
    S = spans[0][1] - spans[0][0]
    n_full = sum(1 for (a, b) in spans if b - a == S)
    sig = np.empty(len(spans), dtype=np.float64)
    sig[:n_full] = s[:, :n_full * S].reshape(nb, n_full, S).max(axis=2).sum(axis=0)
    for j in range(n_full, len(spans)):
        a, b = spans[j]
        sig[j] = s[:, a - mid_lo:b - mid_lo].max(axis=1).sum()
    return sig + 0.0


def _exact_span_score_fractions(q_blk, K_h, qheads, span) -> Fraction:
    """Exact rational span score by direct Fraction arithmetic (slow)."""
    a, b = span
    total = Fraction(0)
    nb, _, d = q_blk.shape
    for i in range(nb):
        best = None
        for t in range(a, b):
            acc = Fraction(0)
            for hq in qheads:
                qv = q_blk[i, hq]
                for c in range(d):
                    acc += Fraction(float(qv[c])) * Fraction(float(K_h[t, c]))
            if best is None or acc > best:
                best = acc
        total += best
    return total


def _lsb_exponent(x: np.ndarray):
    """Largest e such that every element of x is a multiple of 2**e (None if all 0)."""
    nz = x[x != 0]
    if nz.size == 0:
        return None
    m, e = np.frexp(nz)                              # nz = m * 2**e, 0.5 <= |m| < 1
    M = np.abs(np.ldexp(m, 53).astype(np.int64))     # exact integer significand
    low = (M & -M).astype(np.float64)                # lowest set bit, a power of two
    return int(np.min(e - 53 + np.log2(low).astype(np.int64)))


def exact_span_score(q_blk: np.ndarray, K_h: np.ndarray, qheads, span) -> Fraction:
    """Exact rational value of sigma for one span (inputs are dyadic floats).

    Every product is a multiple of u = 2**(lsb(q) + lsb(K)); if every partial sum
    of the token scores and of the block sum is bounded by 2**52 * u, all fp64
    operations on these values are exact and the fp64 evaluation is the exact
    value.  Otherwise the score is evaluated with Fractions.
    """
    a, b = span
    nb, _, d = q_blk.shape
    m = len(qheads)
    Q = q_blk[:, qheads, :].reshape(nb * m, d)
    Ks = K_h[a:b]
    lq, lk = _lsb_exponent(Q), _lsb_exponent(Ks)
    if lq is None or lk is None:
        return Fraction(0)
    unit = 2.0 ** (lq + lk)
    bound = (np.abs(Q) @ np.abs(Ks).T).reshape(nb, m, -1).sum(axis=1) * (1.0 + 1e-9)
    limit = 2.0 ** 52 * unit
    if bound.max() < limit and bound.max(axis=1).sum() * (1.0 + 1e-9) < limit:
        s = (Q @ Ks.T).reshape(nb, m, -1).sum(axis=1)
        return Fraction(float(s.max(axis=1).sum()))
    return _exact_span_score_fractions(q_blk, K_h, qheads, span)


# --------------------------------------------------------------------------
# 5. top-k
# --------------------------------------------------------------------------
def select_topk(sigma: np.ndarray, k: int, exact_fn=None):
    """Indices of the min(k, n) largest sigma, ties -> lower index, ascending.

    `exact_fn(j)` returns the exact score of span j; it is consulted only for
    spans whose fp64 score is within GUARD_REL * max|sigma| of the k-th one.
    """
    n = len(sigma)
    kk = min(max(k, 0), n)
    if kk == 0:
        return []
    if kk == n:
        return list(range(n))
    order = sorted(range(n), key=lambda j: (-sigma[j], j))
    kth = sigma[order[kk - 1]]
    tol = GUARD_REL * max(float(np.abs(sigma).max()), 1e-300)
    band = [j for j in range(n) if abs(sigma[j] - kth) <= tol]
    if len(band) > 1 and exact_fn is not None:
        above = [j for j in range(n) if sigma[j] > kth + tol]
        exact = {j: exact_fn(j) for j in band}
        band_sorted = sorted(band, key=lambda j: (-exact[j], j))
        chosen = above + band_sorted[:kk - len(above)]
    else:
        chosen = order[:kk]
    return sorted(chosen)


def widen_merge(sel_tokens, n_mid: int, S: int):
    """Token-segment selection: every selected token u (middle-relative) is
    widened to the S tokens [u - (S-1)//2, u - (S-1)//2 + S), clipped to the
    middle [0, n_mid); the result is the union, ascending."""
    left = (S - 1) // 2
    cover = set()
    for u in sel_tokens:
        for x in range(u - left, u - left + S):
            if 0 <= x < n_mid:
                cover.add(x)
    return sorted(cover)


# --------------------------------------------------------------------------
# 6-7. window and RoPE
# --------------------------------------------------------------------------
def window_src(T: int, Gp: int, Lp: int, spans, sel):
    """Cache token index of every window row: global ++ selected ++ local."""
    src = list(range(Gp))
    for j in sel:
        a, b = spans[j]
        src.extend(range(a, b))
    src.extend(range(T - Lp, T))
    return np.array(src, dtype=np.int64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE in fp64.  x: [..., d]; pos broadcasts against x[..., 0]."""
    d = x.shape[-1]
    half = d // 2
    inv = np.array([theta ** (-2.0 * c / d) for c in range(half)], dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    cs, sn = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cs - x2 * sn, x2 * cs + x1 * sn], axis=-1)


# --------------------------------------------------------------------------
# 8. attention
# --------------------------------------------------------------------------
def attend_rows(Q: np.ndarray, Kr: np.ndarray, V: np.ndarray, qpos: np.ndarray, scale: float):
    """Rows of softmax attention: row r of the result is
    sum_w softmax_w((Q[r] . Kr[w]) * scale over w <= qpos[r]) * V[w]."""
    logits = (Q @ Kr.T) * scale                                  # [R][W]
    w = np.arange(Kr.shape[0])
    logits = np.where(w[None, :] <= np.asarray(qpos)[:, None], logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# The steps as the library exposes them
# --------------------------------------------------------------------------
def _f64(x):
    return np.asarray(x, dtype=np.float64)


def score_select(q, K, G, S, k, L, block_q=1, return_scores=False, per_q_head=False,
                 token_segments=False):
    """Steps 1-5.  q [n_q][Hq][d], K [Hkv][T][d] (any float dtype, upcast to fp64).

    Returns sel: list over blocks of list over selection units (KV heads, or
    query heads when per_q_head) of ascending span indices (and the fp64 span
    scores [n_blk][n_units][n_spans] if asked).

    token_segments: the k best single tokens are selected instead (their
    scores are the token scores, summed over the block's queries), each is
    widened to a segment of S tokens (widen_merge), and sel holds the union's
    middle-relative token indices; the scores returned are the token scores.
    """
    q = _f64(q)
    K = _f64(K)
    n_q, Hq, d = q.shape
    Hkv, T, _ = K.shape
    units = selection_units(Hq, Hkv, per_q_head)
    Gp, Lp, lo, hi = regions(T, G, L)
    spans = span_list(lo, hi, 1 if token_segments else S)
    n_blk = n_q // block_q
    sel = []
    scores = np.zeros((n_blk, len(units), len(spans)), dtype=np.float64)
    for b in range(n_blk):
        qb = q[b * block_q:(b + 1) * block_q]
        row = []
        for u, (h, qheads) in enumerate(units):
            if spans:
                s = token_scores(qb, K[h], qheads, lo, hi)
                sig = span_scores_from_tokens(s, spans, lo)
            else:
                sig = np.zeros(0)
            scores[b, u] = sig
            chosen = select_topk(
                sig, k,
                lambda j, qb=qb, h=h, qh=qheads: exact_span_score(qb, K[h], qh, spans[j]))
            row.append(widen_merge(chosen, hi - lo, S) if token_segments else chosen)
        sel.append(row)
    return (sel, scores) if return_scores else sel


def gather_rope(q, K, V, sel, G, S, L, block_q=1, theta=500000.0, per_q_head=False,
                token_segments=False):
    """Steps 6-7.  Returns (K_win, V_win, q_rot, W, qpos) with
    K_win/V_win lists [n_blk][n_units] of [W][d] fp64 arrays (K rotated, V
    plain), q_rot [n_q][Hq][d] fp64, W [n_blk][n_units], qpos [n_q][n_units]
    window positions; the units are the KV heads, or the query heads when
    per_q_head (each window is gathered from the unit's KV head).  With
    token_segments, sel holds middle-relative token indices."""
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    n_q, Hq, d = q.shape
    Hkv, T, _ = K.shape
    units = selection_units(Hq, Hkv, per_q_head)
    Gp, Lp, lo, hi = regions(T, G, L)
    spans = span_list(lo, hi, 1 if token_segments else S)
    n_blk = n_q // block_q
    K_win, V_win = [], []
    W = np.zeros((n_blk, len(units)), dtype=np.int64)
    qpos = np.zeros((n_q, len(units)), dtype=np.int64)
    q_rot = np.zeros_like(q)
    for b in range(n_blk):
        kr, vr = [], []
        for u, (h, qheads) in enumerate(units):
            src = window_src(T, Gp, Lp, spans, sel[b][u])
            Wbh = len(src)
            W[b, u] = Wbh
            kr.append(rope(K[h][src], np.arange(Wbh), theta))
            vr.append(V[h][src])
            for i in range(b * block_q, (b + 1) * block_q):
                p_abs = T - n_q + i
                pos = Wbh - (T - p_abs)       # row holding the query's own key
                qpos[i, u] = pos
                q_rot[i, qheads] = rope(q[i, qheads], np.full(len(qheads), pos), theta)
        K_win.append(kr)
        V_win.append(vr)
    return K_win, V_win, q_rot, W, qpos


def window_attend(q_rot, K_win, V_win, qpos, block_q=1, scale=None):
    """Step 8.  Returns out [n_q][Hq][d] fp64.  Unit u of K_win (a KV head, or a
    query head) serves the Hq / n_units consecutive query heads from u * that."""
    n_q, Hq, d = q_rot.shape
    n_units = len(K_win[0])
    m = Hq // n_units
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.zeros((n_q, Hq, d), dtype=np.float64)
    for b in range(n_q // block_q):
        i0, i1 = b * block_q, (b + 1) * block_q
        for u in range(n_units):
            Q = q_rot[i0:i1, u * m:(u + 1) * m].reshape(-1, d)     # rows (i, head)
            pos = np.repeat(qpos[i0:i1, u], m)
            out[i0:i1, u * m:(u + 1) * m] = attend_rows(
                Q, K_win[b][u], V_win[b][u], pos, sc).reshape(i1 - i0, m, d)
    return out


def step(q, K, V, G, S, k, L, block_q=1, theta=500000.0, scale=None, return_all=False,
         per_q_head=False, token_segments=False):
    """Steps 1-8 (the fused decode/prefill step).  Returns (out, sel)."""
    sel = score_select(q, K, G, S, k, L, block_q, per_q_head=per_q_head,
                       token_segments=token_segments)
    K_win, V_win, q_rot, W, qpos = gather_rope(q, K, V, sel, G, S, L, block_q, theta,
                                               per_q_head=per_q_head,
                                               token_segments=token_segments)
    out = window_attend(q_rot, K_win, V_win, qpos, block_q, scale)
    if return_all:
        return dict(out=out, sel=sel, K_win=K_win, V_win=V_win, q_rot=q_rot, W=W, qpos=qpos)
    return out, sel
