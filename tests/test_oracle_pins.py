"""Pins for the CPU oracle: each checks it against something other than itself.

  * hand-worked integer cases (tests/golden/hand_worked.json)
  * closed-form region/span/window sizes of the evaluation workloads and of the
    pages' own LLaMA3-8B-8K setting (global 32 + 127 spans x 32 + local 4096 =
    the model's 8192 trained positions)
  * special cases that reduce to textbook attention (torch's
    scaled_dot_product_attention, RoPE written as a complex rotation)
  * brute force over all k-subsets on tiny inputs
  * a second scalar coding with exact rational span scores (tests/scalar_twin.py)
  * RoPE invariants, needle recall, invariance to unselected spans
  * mutation tests: plausible mistakes planted in the oracle must fail a pin
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.rea_oracle as O
from tests import scalar_twin

HERE = os.path.dirname(os.path.abspath(__file__))
THETA = 500000.0


# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------
def rope_complex(x, pos, theta=THETA):
    """RoPE as a complex rotation of (x_c + i x_{c+d/2}) by pos * theta^(-2c/d)."""
    x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    d = x.shape[-1]
    half = d // 2
    freq = torch.tensor([theta ** (-2.0 * c / d) for c in range(half)], dtype=torch.float64)
    ang = torch.as_tensor(np.asarray(pos, dtype=np.float64))[..., None] * freq
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def sdpa_ref(q, keys, vals, key_pos, q_pos, theta=THETA):
    """Textbook causal attention: q [n][Hq][d], keys/vals [Hkv][W][d] with
    positions key_pos [W]; query i attends to keys with key_pos <= q_pos[i]."""
    q = np.asarray(q, dtype=np.float64)
    n, Hq, d = q.shape
    Hkv = keys.shape[0]
    g = Hq // Hkv
    kr = rope_complex(keys, key_pos[None, :].repeat(Hkv, 0), theta)          # [Hkv][W][d]
    qr = rope_complex(q, np.repeat(np.asarray(q_pos)[:, None], Hq, 1), theta)  # [n][Hq][d]
    kr = kr.repeat_interleave(g, dim=0)                                     # [Hq][W][d]
    vv = torch.as_tensor(np.asarray(vals, dtype=np.float64)).repeat_interleave(g, dim=0)
    mask = torch.as_tensor(np.asarray(key_pos)[None, :] <= np.asarray(q_pos)[:, None])  # [n][W]
    out = torch.nn.functional.scaled_dot_product_attention(
        qr.permute(1, 0, 2), kr, vv, attn_mask=mask[None].expand(Hq, -1, -1))
    return out.permute(1, 0, 2).numpy()


def rand_problem(rng, n_q, Hq, Hkv, d, T, kind="bf16"):
    if kind == "int":
        q = rng.integers(-2, 3, size=(n_q, Hq, d)).astype(np.float64)
        K = rng.integers(-2, 3, size=(Hkv, T, d)).astype(np.float64)
        V = rng.integers(-2, 3, size=(Hkv, T, d)).astype(np.float64)
        return q, K, V
    q = rng.standard_normal((n_q, Hq, d)).astype(np.float32)
    K = rng.standard_normal((Hkv, T, d)).astype(np.float32)
    V = rng.standard_normal((Hkv, T, d)).astype(np.float32)
    if kind == "bf16":   # truncate to bf16-representable values
        q, K, V = [(a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32) for a in (q, K, V)]
    return q.astype(np.float64), K.astype(np.float64), V.astype(np.float64)


def load_golden():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


# --------------------------------------------------------------------------
# pin checks (each returns None or raises AssertionError); reused by mutations
# --------------------------------------------------------------------------
def check_golden():
    for case in load_golden():
        q = np.array(case["q"], dtype=np.float64)
        K = np.array(case["K"], dtype=np.float64)
        V = K.copy()
        G, S, L, bq = case["G"], case["S"], case["L"], case["block_q"]
        pqh = case.get("per_q_head", False)
        tseg = case.get("token_segments", False)
        Hkv, T, _ = K.shape
        g = q.shape[1] // Hkv
        for ex in case["expect"]:
            sel, sc = O.score_select(q, K, G, S, ex["k"], L, bq, return_scores=True,
                                     per_q_head=pqh, token_segments=tseg)
            assert sel == ex["sel"], (case["name"], ex["k"], sel)
            exp_sc = np.array(case["span_scores"], dtype=np.float64)
            assert sc.shape == exp_sc.shape and np.array_equal(sc, exp_sc), (case["name"], sc)
            Kw, Vw, qr, W, qpos = O.gather_rope(q, K, V, sel, G, S, L, bq, per_q_head=pqh,
                                                token_segments=tseg)
            assert W.tolist() == ex["W"], (case["name"], W)
            assert qpos.tolist() == ex["qpos"], (case["name"], qpos)
            for b in range(len(sel)):
                for u in range(len(sel[b])):
                    h = u // g if pqh else u
                    src = np.array(ex["src"][b][u])
                    assert np.array_equal(Vw[b][u], V[h][src]), (case["name"], "V window")


def check_full_attention(seed=1):
    """All spans selected (T <= G + k*S + L, or k >= n_spans): the window is the
    whole cache and the result is plain causal RoPE attention."""
    rng = np.random.default_rng(seed)
    for (n_q, bq, Hq, Hkv, d, T, G, S, k, L) in [
            (1, 1, 4, 2, 8, 37, 3, 4, 8, 6),      # T <= G+kS+L, partial last span
            (1, 1, 2, 1, 16, 90, 2, 8, 100, 5),   # k >> n_spans
            (4, 2, 2, 2, 8, 40, 1, 5, 9, 8)]:     # prefill blocks
        q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T)
        out, sel = O.step(q, K, V, G, S, k, L, bq)
        pos = np.arange(T)
        ref = sdpa_ref(q, K, V, pos, pos[T - n_q:])
        np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def check_k0(seed=2):
    """k = 0: attention over the global and local caches only, positions
    0..G'+L'-1 (the StreamingLLM-style sink + local window)."""
    rng = np.random.default_rng(seed)
    n_q, Hq, Hkv, d, T, G, S, L = 2, 4, 2, 8, 60, 3, 4, 7
    q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T)
    out, sel = O.step(q, K, V, G, S, 0, L, block_q=1)
    idx = np.r_[0:G, T - L:T]
    pos = np.arange(len(idx))
    ref = sdpa_ref(q, K[:, idx], V[:, idx], pos, pos[len(idx) - n_q:])
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def check_bruteforce(seed=3):
    """Top-k against an enumeration of every k-subset: the selected set must be
    the one whose every member beats every non-member under (score, -index)."""
    rng = np.random.default_rng(seed)
    for trial in range(6):
        kind = "int" if trial % 2 else "bf16"
        Hq, Hkv, d, S = 2, 1, 4, 3
        n_sp = int(rng.integers(4, 9))
        G, L = 2, 3
        T = G + L + n_sp * S - int(rng.integers(0, S))   # maybe a partial last span
        q, K, V = rand_problem(rng, 1, Hq, Hkv, d, T, kind)
        lo, hi = G, T - L
        spans = [(a, min(a + S, hi)) for a in range(lo, hi, S)]
        exact = [max(sum(Fraction(float(q[0, gg, c])) * Fraction(float(K[0, t, c]))
                         for gg in range(Hq) for c in range(d))
                     for t in range(a, b)) for (a, b) in spans]
        for k in range(0, 5):
            good = []
            for sub in itertools.combinations(range(len(spans)), min(k, len(spans))):
                rest = [j for j in range(len(spans)) if j not in sub]
                if all((exact[a], -a) > (exact[b], -b) for a in sub for b in rest):
                    good.append(sorted(sub))
            assert len(good) == 1
            sel = O.score_select(q, K, G, S, k, L)
            assert sel[0][0] == good[0], (trial, k, sel, good)


def check_scalar_twin(seed=4):
    """numpy oracle == scalar exact-rational twin on tiny inputs."""
    rng = np.random.default_rng(seed)
    shapes = [  # n_q, bq, Hq, Hkv, d, T, G, S, k, L, kind
        (1, 1, 4, 2, 4, 29, 2, 3, 3, 4, "bf16"),
        (1, 1, 2, 1, 6, 31, 1, 4, 2, 5, "int"),
        (4, 2, 2, 1, 4, 26, 2, 3, 2, 6, "f32"),
        (2, 1, 3, 1, 4, 19, 0, 2, 3, 3, "int"),
        (1, 1, 2, 2, 4, 11, 4, 2, 1, 8, "bf16"),     # T <= G+L
    ]
    per_head_shapes = [
        (1, 1, 4, 2, 4, 29, 2, 3, 3, 4, "bf16"),
        (2, 2, 3, 1, 4, 23, 1, 2, 2, 5, "int"),
        (1, 1, 2, 1, 4, 21, 2, 1, 5, 3, "f32"),      # token level (S = 1)
    ]
    segment_shapes = [
        (1, 1, 4, 2, 4, 37, 2, 3, 3, 4, "bf16"),
        (2, 2, 2, 1, 4, 31, 1, 4, 2, 5, "int"),      # ties, blocks, even width
        (1, 1, 2, 1, 4, 26, 2, 5, 4, 3, "f32"),      # overlapping and clipped segments
    ]
    cases = ([(sh, False, False) for sh in shapes] + [(sh, True, False) for sh in per_head_shapes]
             + [(sh, False, True) for sh in segment_shapes])
    for (n_q, bq, Hq, Hkv, d, T, G, S, k, L, kind), pqh, tseg in cases:
        q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T, kind)
        out_tw, sel_tw, W_tw = scalar_twin.step(q.tolist(), K.tolist(), V.tolist(), G, S, k, L, bq,
                                                per_q_head=pqh, token_segments=tseg)
        res = O.step(q, K, V, G, S, k, L, bq, return_all=True, per_q_head=pqh,
                     token_segments=tseg)
        assert res["sel"] == sel_tw, (res["sel"], sel_tw)
        assert res["W"].tolist() == W_tw
        np.testing.assert_allclose(res["out"], np.array(out_tw), rtol=1e-9, atol=1e-12)


def check_per_q_head_is_repeated_kv(seed=7):
    """Selecting per query head equals selecting per KV head on a cache whose
    KV heads are repeated once per query head (group size 1): same span
    scores, selections, windows and outputs."""
    rng = np.random.default_rng(seed)
    for (n_q, bq, Hq, Hkv, d, T, G, S, k, L, kind) in [
            (1, 1, 4, 2, 8, 70, 3, 4, 5, 6, "bf16"),
            (4, 2, 6, 2, 8, 61, 2, 3, 4, 9, "int"),
            (1, 1, 3, 1, 4, 40, 1, 1, 9, 4, "f32")]:
        q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T, kind)
        g = Hq // Hkv
        Kr, Vr = np.repeat(K, g, axis=0), np.repeat(V, g, axis=0)
        a = O.step(q, K, V, G, S, k, L, bq, return_all=True, per_q_head=True)
        b = O.step(q, Kr, Vr, G, S, k, L, bq, return_all=True)
        assert a["sel"] == b["sel"]
        assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["qpos"], b["qpos"])
        np.testing.assert_array_equal(a["out"], b["out"])
        _, sa = O.score_select(q, K, G, S, k, L, bq, return_scores=True, per_q_head=True)
        _, sb = O.score_select(q, Kr, G, S, k, L, bq, return_scores=True)
        np.testing.assert_array_equal(sa, sb)


def check_needle(seed=5):
    """A span whose keys point along the group's query sum is recalled, and
    shuffling spans that were not selected changes nothing."""
    rng = np.random.default_rng(seed)
    n_q, Hq, Hkv, d, T, G, S, k, L = 1, 4, 2, 16, 400, 4, 8, 4, 32
    q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T, "f32")
    lo = G
    needle = {0: 17, 1: 30}
    for h, j in needle.items():
        qe = q[0, h * 2:(h + 1) * 2].sum(axis=0)
        K[h, lo + j * S:lo + (j + 1) * S] = qe + 0.1 * rng.standard_normal((S, d))
    out, sel = O.step(q, K, V, G, S, k, L)
    for h, j in needle.items():
        assert j in sel[0][h], (h, sel)
    n_sp = (T - L - G) // S
    K2, V2 = K.copy(), V.copy()
    for h in range(Hkv):
        free = [j for j in range(n_sp) if j not in sel[0][h]]
        perm = rng.permutation(free)
        for a, b in zip(free, perm):
            K2[h, lo + a * S:lo + (a + 1) * S] = K[h, lo + b * S:lo + (b + 1) * S]
            V2[h, lo + a * S:lo + (a + 1) * S] = V[h, lo + b * S:lo + (b + 1) * S]
    out2, sel2 = O.step(q, K2, V2, G, S, k, L)
    assert sel2 == sel
    np.testing.assert_array_equal(out2, out)


def check_rope():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 32))
    y = rng.standard_normal((5, 32))
    np.testing.assert_array_equal(O.rope(x, np.zeros(5), THETA), x)
    p = np.array([0, 3, 77, 1000, 8191])
    rx = O.rope(x, p, THETA)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(rx, rope_complex(x, p).numpy(), rtol=1e-12, atol=1e-12)
    # relative: <R(p)x, R(p')y> depends on p - p' only
    a = (O.rope(x, p, THETA) * O.rope(y, p + 5, THETA)).sum(1)
    b = (O.rope(x, p + 1234, THETA) * O.rope(y, p + 1239, THETA)).sum(1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def check_token_segments(seed=8):
    """Token segments of width 1 are token-level span selection; every
    selected token's segment lies in the union, which holds at most k*S
    tokens; selecting every token gives full attention."""
    rng = np.random.default_rng(seed)
    for (n_q, bq, Hq, Hkv, d, T, G, S, k, L) in [(1, 1, 4, 2, 8, 90, 3, 5, 6, 7),
                                                (4, 2, 2, 1, 8, 70, 2, 4, 5, 6)]:
        q, K, V = rand_problem(rng, n_q, Hq, Hkv, d, T)
        a = O.step(q, K, V, G, 1, k, L, bq, return_all=True, token_segments=True)
        b = O.step(q, K, V, G, 1, k, L, bq, return_all=True)
        assert a["sel"] == b["sel"]
        np.testing.assert_array_equal(a["out"], b["out"])
        sel_tok = O.score_select(q, K, G, 1, k, L, bq)
        seg = O.score_select(q, K, G, S, k, L, bq, token_segments=True)
        n_mid = T - G - L
        for blk in range(len(seg)):
            for h in range(Hkv):
                u = set(seg[blk][h])
                assert len(u) <= k * S and seg[blk][h] == sorted(u)
                for t in sel_tok[blk][h]:
                    lo = t - (S - 1) // 2
                    assert all(x in u for x in range(max(lo, 0), min(lo + S, n_mid)))
        out, _ = O.step(q, K, V, G, S, T, L, bq, token_segments=True)
        pos = np.arange(T)
        np.testing.assert_allclose(out, sdpa_ref(q, K, V, pos, pos[T - n_q:]), rtol=1e-10,
                                   atol=1e-12)


PINS = [check_golden, check_full_attention, check_k0, check_bruteforce,
        check_scalar_twin, check_needle, check_rope, check_per_q_head_is_repeated_kv,
        check_token_segments]


# --------------------------------------------------------------------------
# the pins as tests
# --------------------------------------------------------------------------
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_region_closed_forms():
    # tiny fp32 workload: T 4096, G 4, S 16, L 64 -> middle 4028 tokens, 252 spans, last 12
    Gp, Lp, lo, hi = O.regions(4096, 4, 64)
    sp = O.span_list(lo, hi, 16)
    assert (lo, hi, len(sp), sp[-1][1] - sp[-1][0]) == (4, 4032, 252, 12)
    # 8B decode at 128K: 126944 middle tokens = 3967 spans of 32
    _, _, lo, hi = O.regions(131072, 32, 4096)
    assert (hi - lo, len(O.span_list(lo, hi, 32))) == (126944, 3967)
    # 8B prefill chunk: 4096 new tokens appended at 131072 -> 4095 spans
    _, _, lo, hi = O.regions(131072 + 4096, 32, 4096)
    assert len(O.span_list(lo, hi, 32)) == 4095
    # 3B decode at 4M, S 64: 65286 spans, the last one 32 tokens
    _, _, lo, hi = O.regions(4194304, 32, 16000)
    sp = O.span_list(lo, hi, 64)
    assert (len(sp), sp[-1][1] - sp[-1][0]) == (65286, 32)
    # the pages' LLaMA3-8B-8K setting fills exactly the 8192 trained positions
    assert 32 + 127 * 32 + 4096 == 8192
    # degenerate: T <= G + L -> no middle
    assert O.regions(5, 2, 4) == (2, 3, 2, 2)
    assert O.regions(3, 8, 4) == (3, 0, 3, 3)


def test_window_size_bound():
    """W = G' + (selected tokens) + L' <= G + k*S + L, with equality when
    every selected span is full."""
    rng = np.random.default_rng(11)
    q, K, V = rand_problem(rng, 1, 2, 1, 8, 203, "f32")
    for k in range(0, 30, 3):
        sel = O.score_select(q, K, 5, 7, k, 11)
        _, _, _, W, _ = O.gather_rope(q, K, V, sel, 5, 7, 11)
        n_full = sum(1 for j in sel[0][0] if j < 26)   # middle 187 = 26 x 7 + 5
        partial = 5 if 26 in sel[0][0] else 0
        assert W[0, 0] == 5 + 7 * n_full + partial + 11 <= 5 + k * 7 + 11


def test_exact_guard_resolves_near_tie():
    """Two spans whose exact scores differ by 2^-40 relative: fp64 rounding of
    the sum can hide the gap, the Fraction guard must not."""
    d = 4
    q = np.array([[[1.0, 1.0, 1.0, 1.0]]])
    big = 2.0 ** 20
    K = np.zeros((1, 12, d))
    # spans [1,3) [3,5) [5,7): exact scores big + 2^-35, big + 2^-33, big + 2^-34;
    # in fp64 all three round to big, so only the exact guard finds span 1
    K[0, 1] = [big, 2.0 ** -35, 0, 0]
    K[0, 3] = [big, 2.0 ** -33, 0, 0]
    K[0, 5] = [big, 2.0 ** -34, 0, 0]
    sel, sc = O.score_select(q, K, 1, 2, 1, 5, return_scores=True)
    assert np.all(sc == big)
    assert sel == [[[1]]]
    sig = np.array([3.0, 3.0, 3.0])
    assert O.select_topk(sig, 2, lambda j: [1, 3, 2][j]) == [1, 2]


def test_exact_score_fast_path_matches_fractions():
    """The fp64-is-exact shortcut of the tie guard equals Fraction arithmetic,
    and falls back to it when the exponent spread is too wide."""
    rng = np.random.default_rng(12)
    for kind in ("bf16", "int", "f32"):
        q, K, V = rand_problem(rng, 3, 4, 2, 8, 40, kind)
        for h in range(2):
            for span in [(3, 9), (10, 11), (20, 40)]:
                fast = O.exact_span_score(q, K[h], [2 * h, 2 * h + 1], span)
                slow = O._exact_span_score_fractions(q, K[h], [2 * h, 2 * h + 1], span)
                assert fast == slow, (kind, h, span)
                fast = O.exact_span_score(q, K[h], [2 * h + 1], span)
                slow = O._exact_span_score_fractions(q, K[h], [2 * h + 1], span)
                assert fast == slow, (kind, h, span)
    # spread of 2^80 between terms: fp64 cannot hold the sum, Fractions must be used
    q = np.array([[[1.0, 1.0]]])
    K = np.array([[2.0 ** 40, 2.0 ** -40]])
    assert O.exact_span_score(q, K, [0], (0, 1)) == Fraction(2 ** 40) + Fraction(1, 2 ** 40)
    assert O._lsb_exponent(np.array([0.75, 3.0, 0.0])) == -2


# --------------------------------------------------------------------------
# mutation tests: a planted mistake must fail at least one pin
# --------------------------------------------------------------------------
def _mut_span_sum(s, spans, mid_lo):
    sig = np.array([s[:, a - mid_lo:b - mid_lo].sum(axis=1).sum() for (a, b) in spans])
    return sig + 0.0


def _mut_span_max_of_sum(s, spans, mid_lo):
    return np.array([s[:, a - mid_lo:b - mid_lo].sum(axis=0).max() for (a, b) in spans]) + 0.0


_orig_token_scores = O.token_scores
_orig_select = O.select_topk
_orig_rope = O.rope
_orig_attend = O.attend_rows
_orig_regions = O.regions
_orig_span_list = O.span_list


_orig_units = O.selection_units
_orig_widen = O.widen_merge


def _mut_widen_left_heavy(sel_tokens, n_mid, S):
    return _orig_widen([u + ((S - 1) // 2) - S // 2 for u in sel_tokens], n_mid, S)


def _mut_widen_no_clip(sel_tokens, n_mid, S):
    return _orig_widen(sel_tokens, n_mid + S, S)


def _mut_first_head(q_blk, K_h, qheads, lo, hi):
    return q_blk[:, qheads[0], :] @ K_h[lo:hi].T


def _mut_wrong_head(q_blk, K_h, qheads, lo, hi):
    Hq, m = q_blk.shape[1], len(qheads)
    return _orig_token_scores(q_blk, K_h, [(hq + m) % Hq for hq in qheads], lo, hi)


def _mut_per_head_kv_modulo(Hq, Hkv, per_q_head=False):
    if per_q_head:
        return [(hq % Hkv, [hq]) for hq in range(Hq)]
    return _orig_units(Hq, Hkv, per_q_head)


def _mut_per_head_sums_group(Hq, Hkv, per_q_head=False):
    units = _orig_units(Hq, Hkv, False)
    if per_q_head:
        g = Hq // Hkv
        return [units[hq // g] for hq in range(Hq)]
    return units


def _mut_tie_high(sigma, k, exact_fn=None):
    n = len(sigma)
    kk = min(k, n)
    order = sorted(range(n), key=lambda j: (-sigma[j], -j))
    return sorted(order[:kk])


def _mut_unsorted(sigma, k, exact_fn=None):
    n = len(sigma)
    order = sorted(range(n), key=lambda j: (-sigma[j], j))
    return order[:min(k, n)]


def _mut_rope_sign(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    inv = np.array([theta ** (-2.0 * c / d) for c in range(half)])
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * np.cos(ang) + x2 * np.sin(ang),
                           x2 * np.cos(ang) + x1 * np.sin(ang)], axis=-1)


def _mut_rope_adjacent_pairs(x, pos, theta):
    d = x.shape[-1]
    perm = np.r_[0:d:2, 1:d:2]
    inv_perm = np.argsort(perm)
    return _orig_rope(x[..., perm], pos, theta)[..., inv_perm]


def _mut_no_scale(Q, Kr, V, qpos, scale):
    return _orig_attend(Q, Kr, V, qpos, 1.0)


def _mut_exclude_self(Q, Kr, V, qpos, scale):
    return _orig_attend(Q, Kr, V, np.maximum(np.asarray(qpos) - 1, 0), scale)


def _mut_local_short(T, G, L):
    Gp, Lp, lo, hi = _orig_regions(T, G, L)
    if Lp > 1:
        return Gp, Lp - 1, lo, hi + 1
    return Gp, Lp, lo, hi


def _mut_drop_partial(lo, hi, S):
    return [sp for sp in _orig_span_list(lo, hi, S) if sp[1] - sp[0] == S]


MUTATIONS = {
    "span_sum_not_max": ("span_scores_from_tokens", _mut_span_sum),
    "block_max_of_sums": ("span_scores_from_tokens", _mut_span_max_of_sum),
    "gqa_first_head_only": ("token_scores", _mut_first_head),
    "gqa_wrong_group": ("token_scores", _mut_wrong_head),
    "per_q_head_kv_by_modulo": ("selection_units", _mut_per_head_kv_modulo),
    "per_q_head_scores_whole_group": ("selection_units", _mut_per_head_sums_group),
    "segment_extra_token_on_the_left": ("widen_merge", _mut_widen_left_heavy),
    "segment_not_clipped_to_middle": ("widen_merge", _mut_widen_no_clip),
    "ties_to_higher_index": ("select_topk", _mut_tie_high),
    "spans_in_score_order": ("select_topk", _mut_unsorted),
    "rope_sign_flip": ("rope", _mut_rope_sign),
    "rope_adjacent_pairing": ("rope", _mut_rope_adjacent_pairs),
    "no_softmax_scale": ("attend_rows", _mut_no_scale),
    "query_excludes_own_key": ("attend_rows", _mut_exclude_self),
    "local_region_short_by_one": ("regions", _mut_local_short),
    "partial_span_dropped": ("span_list", _mut_drop_partial),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
