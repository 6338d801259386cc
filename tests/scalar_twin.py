"""Second, independent coding of the ReAttention hot path in scalar Python.

Every loop is written out; span scores and the top-k decision use exact
rational arithmetic (fractions.Fraction), so on tiny inputs this is the exact
definition.  It shares no code with oracle/ and is used to pin it.
"""
import math
from fractions import Fraction


def _rot(x, pos, theta):
    d = len(x)
    half = d // 2
    y = [0.0] * d
    for c in range(half):
        ang = pos * (theta ** (-2.0 * c / d))
        cs, sn = math.cos(ang), math.sin(ang)
        y[c] = x[c] * cs - x[c + half] * sn
        y[c + half] = x[c + half] * cs + x[c] * sn
    return y


def step(q, K, V, G, S, k, L, block_q=1, theta=500000.0, scale=None, per_q_head=False,
         token_segments=False):
    """q [n_q][Hq][d], K/V [Hkv][T][d] as nested lists of floats.

    Returns (out [n_q][Hq][d] floats, sel [n_blk][units] lists, W [n_blk][units]),
    where the units are the KV heads (each scored with its group's summed
    logits) or, with per_q_head, the query heads (each with its own logits
    against its group's KV head).  token_segments: the k best single tokens,
    each widened to S tokens around it (from u - (S-1)//2), clipped to the
    middle and joined; sel then lists middle-relative tokens.
    """
    n_q, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv, T = len(K), len(K[0])
    g = Hq // Hkv
    Gp = min(G, T)
    Lp = min(L, T - Gp)
    lo, hi = Gp, T - Lp
    width = 1 if token_segments else S
    spans = []
    a = lo
    while a < hi:
        spans.append((a, min(a + width, hi)))
        a += width
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(n_q)]
    sel_all, W_all = [], []
    if per_q_head:
        units = []
        for hq in range(Hq):
            units.append((hq // g, [hq]))
    else:
        units = []
        for h in range(Hkv):
            units.append((h, [h * g + gg for gg in range(g)]))
    for b in range(n_q // block_q):
        sel_b, W_b = [], []
        for (h, heads) in units:
            sig = []
            for (a, e) in spans:
                tot = Fraction(0)
                for i in range(b * block_q, (b + 1) * block_q):
                    best = None
                    for t in range(a, e):
                        acc = Fraction(0)
                        for hq in heads:
                            for c in range(d):
                                acc += Fraction(q[i][hq][c]) * Fraction(K[h][t][c])
                        if best is None or acc > best:
                            best = acc
                    tot += best
                sig.append(tot)
            remaining = list(range(len(spans)))
            chosen = []
            for _ in range(min(k, len(spans))):
                bj = remaining[0]
                for j in remaining[1:]:
                    if sig[j] > sig[bj]:      # strict: equal scores keep the lower index
                        bj = j
                chosen.append(bj)
                remaining.remove(bj)
            chosen.sort()
            if token_segments:
                # walk the tokens in order, extending the current run of the
                # union or starting a new one
                runs = []
                for u in chosen:
                    a0 = max(u - (S - 1) // 2, 0)
                    a1 = min(u - (S - 1) // 2 + S, hi - lo)
                    if runs and a0 <= runs[-1][1]:
                        runs[-1][1] = max(runs[-1][1], a1)
                    else:
                        runs.append([a0, a1])
                chosen = [x for (r0, r1) in runs for x in range(r0, r1)]
            src = list(range(Gp))
            for j in chosen:
                src += list(range(spans[j][0], spans[j][1]))
            src += list(range(T - Lp, T))
            Wh = len(src)
            krot = [_rot(K[h][src[w]], w, theta) for w in range(Wh)]
            for i in range(b * block_q, (b + 1) * block_q):
                pos = Wh - n_q + i
                for hq in heads:
                    qr = _rot(q[i][hq], pos, theta)
                    logits = []
                    for w in range(pos + 1):
                        s = 0.0
                        for c in range(d):
                            s += qr[c] * krot[w][c]
                        logits.append(s * sc)
                    m = max(logits)
                    p = [math.exp(x - m) for x in logits]
                    z = sum(p)
                    for c in range(d):
                        acc = 0.0
                        for w in range(pos + 1):
                            acc += p[w] * V[h][src[w]][c]
                        out[i][hq][c] = acc / z
            sel_b.append(chosen)
            W_b.append(Wh)
        sel_all.append(sel_b)
        W_all.append(W_b)
    return out, sel_all, W_all
