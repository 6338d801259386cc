"""GPU parity: the library (through its C ABI) against the fp64 oracle on the
same seeded inputs.  Selection must match exactly, window lengths and value
rows bit-exactly, rotated rows to fp32 rounding, outputs within the stated
max-abs tolerance (2e-2 for bf16 inputs, 1e-5 for fp32)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from synth import torch_io
from tests.parity import (TOL, compare_head, device_inputs, log, oracle_head,
                          run_library)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def S(**kw):
    return synth.small(**kw)


SMALL = {
    "bf16_g2_d64_partial": S(),
    "f32_g1_d128_partial": S(dtype="f32", Hq=2, Hkv=2, d=128, T=1010, S=32, topk=7, L=100),
    "bf16_k0": S(topk=0, T=500),
    "bf16_all_spans": S(T=300, S=16, topk=50),
    "bf16_no_middle": S(T=50, G=4, L=64),
    "bf16_prefill_blocks": S(Hq=8, Hkv=2, d=128, T=600, n_q=8, block_q=4, S=16, topk=6,
                             L=64, needles=0),
    "f32_prefill_blocks": S(dtype="f32", Hq=4, Hkv=1, d=64, T=900, n_q=16, block_q=16, S=32,
                            topk=3, L=40, needles=0),
    "bf16_G0": S(G=0, T=800),
    "bf16_token_level_S1": S(S=1, topk=40, T=400),
    "bf16_S20": S(S=20, topk=9, T=1500, kv_scaled=True),
    "bf16_S64_g8": S(Hq=8, Hkv=1, d=128, S=64, topk=6, T=3000, L=200, needles=2),
    "f32_L1": S(dtype="f32", L=1, T=400, topk=4),
    "bf16_many_heads": S(Hq=32, Hkv=8, d=128, T=2048, S=32, topk=12, L=256, needles=2,
                         kv_scaled=True),
    # 3 query heads per KV head (the 3B shape's group): 3 query rows in the
    # fused decode attention
    "bf16_g3_d128": S(Hq=6, Hkv=2, d=128, T=3000, S=32, topk=12, L=256, needles=2,
                      kv_scaled=True),
    # blocks of 64 bf16 queries, d 128: scored on MFMA, certified top-k
    "bf16_mfma_blocks": S(Hq=8, Hkv=2, d=128, T=3000, n_q=128, block_q=64, S=32, topk=12,
                          L=128, needles=0),
    "bf16_mfma_S64_partial": S(Hq=8, Hkv=2, d=128, T=5000, n_q=64, block_q=64, S=64, topk=9,
                               L=100, needles=0, kv_scaled=True),
    "bf16_mfma_5_blocks_g1": S(Hq=2, Hkv=2, d=128, T=2500, n_q=320, block_q=64, S=32, topk=7,
                               L=400, needles=0),
    # 16 blocks x 8 KV heads = 128 pairs: the certification's re-scoring on 8
    # workgroups per pair (the small cases above take 16)
    "bf16_mfma_128_pairs": S(Hq=32, Hkv=8, d=128, T=6000, n_q=1024, block_q=64, S=32, topk=10,
                             L=1024, needles=0, kv_scaled=True),
    # one selection per query head
    "pqh_bf16_g4_d128": S(Hq=8, Hkv=2, d=128, T=2048, S=32, topk=12, L=256, needles=2,
                          kv_scaled=True, per_q_head=True),
    "pqh_f32_g2_partial": S(dtype="f32", per_q_head=True),
    "pqh_bf16_g3_S16": S(Hq=6, Hkv=2, d=128, T=1500, S=16, topk=9, L=100, per_q_head=True),
    "pqh_bf16_g8_d64": S(Hq=8, Hkv=1, d=64, T=1800, S=32, topk=10, L=128, per_q_head=True),
    "pqh_bf16_g5_generic": S(Hq=10, Hkv=2, d=64, T=900, S=16, topk=6, L=64, per_q_head=True),
    "pqh_bf16_token_level": S(S=1, topk=40, T=400, per_q_head=True),
    # one selection per query head past 4096 spans: MFMA scoring, candidate
    # spans, certification with the single-query fp64 re-scoring
    "pqh_bf16_g4_d128_past_4096_spans": S(Hq=8, Hkv=2, d=128, T=200000, S=32, topk=40, L=256,
                                          needles=2, kv_scaled=True, per_q_head=True),
    "pqh_bf16_g2_d128_S64_partial": S(Hq=4, Hkv=2, d=128, T=9000, S=64, topk=11, L=300,
                                      needles=1, per_q_head=True),
    "pqh_bf16_g2_d128_S20": S(Hq=4, Hkv=2, d=128, T=1500, S=20, topk=9, L=100,
                              kv_scaled=True, per_q_head=True),
    "pqh_f32_g4_d64_S8": S(dtype="f32", Hq=8, Hkv=2, d=64, T=1300, S=8, topk=17, L=90,
                           per_q_head=True),
    "pqh_bf16_prefill_blocks": S(Hq=8, Hkv=2, d=128, T=600, n_q=8, block_q=4, S=16, topk=6,
                                 L=64, needles=0, per_q_head=True),
    "pqh_bf16_mfma_blocks": S(Hq=8, Hkv=2, d=128, T=3000, n_q=128, block_q=64, S=32, topk=12,
                              L=128, needles=0, per_q_head=True),
    "f32_token_level_S1_g1": S(dtype="f32", Hq=2, Hkv=2, d=128, S=1, topk=100, T=1200, L=50),
    # bf16 rows of 128: the token scorer's paired-row layout (half rows of two
    # rows per load), 1446 middle tokens (a last group of 6); one, three and
    # four query heads scored per read of a key row
    "bf16_d128_token_level": S(Hq=8, Hkv=2, d=128, S=1, topk=60, T=1500, L=50, needles=2),
    "pqh_bf16_d128_g3_token_level": S(Hq=6, Hkv=2, d=128, S=1, topk=60, T=1500, L=50,
                                      needles=2, per_q_head=True),
    "pqh_bf16_d128_g4_token_level": S(Hq=8, Hkv=2, d=128, S=1, topk=60, T=1500, L=50,
                                      needles=2, per_q_head=True),
    # 9..64 query rows per (block, selection head): 2-wave MFMA attention
    "bf16_blocks_of_16_rows_S24": S(Hq=8, Hkv=2, d=128, T=1900, n_q=8, block_q=4, S=24, topk=9,
                                    L=96, needles=0, kv_scaled=True),
    "pqh_bf16_blocks_64_rows": S(Hq=8, Hkv=2, d=128, T=3000, n_q=128, block_q=64, S=32, topk=12,
                                 L=128, needles=0, per_q_head=True),
    # token level over more than 32768 groups of 32 tokens: the top-k's large
    # path streams the group maxima instead of holding them in registers
    "bf16_token_level_33k_groups": S(Hq=2, Hkv=1, d=64, T=1_060_000, S=1, topk=300, L=64,
                                     needles=2),
    # token level with 32,498 groups: the group maxima held in registers, a
    # contiguous chunk of 4096 per wave; the last wave's chunk holds 3826 (its
    # last lanes ragged) and the last group 28 tokens
    "bf16_token_level_32k_groups": S(Hq=2, Hkv=1, d=64, T=1_040_000, S=1, topk=300, L=64,
                                     needles=2),
    # 65536 spans in 2048 groups, k = 256, needles stretching the score
    # range: the top-k's first bound keeps more groups than it can hold, so
    # the bound becomes the 256-th largest group maximum
    "bf16_k256_2048_groups": S(Hq=2, Hkv=1, d=64, T=262_144, S=4, topk=256, L=64, needles=4),
    # at most 4096 spans (2185 here) with k = 300: the top-k holds every
    # span score in registers, and more than 192 of them reach its bound, so
    # the cutoff comes from histogram levels and the output from a bitmap
    "bf16_k300_2185_spans": S(Hq=4, Hkv=2, d=64, T=70_000, S=32, topk=300, L=64, needles=2),
    # token segments: the best tokens, each widened to S tokens
    "seg_bf16_d64": S(S=8, topk=6, T=700, token_segments=True),
    "seg_bf16_d128_pqh": S(Hq=8, Hkv=2, d=128, T=2048, S=32, topk=12, L=256, needles=2,
                           per_q_head=True, token_segments=True),
    "seg_f32_blocks_S5": S(dtype="f32", Hq=4, Hkv=1, d=64, T=900, n_q=16, block_q=16, S=5,
                           topk=7, L=40, needles=0, token_segments=True),
    "seg_bf16_blocks_mfma_attention": S(Hq=8, Hkv=2, d=128, T=3000, n_q=128, block_q=64, S=32,
                                        topk=12, L=128, needles=0, token_segments=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small(name):
    w = SMALL[name]
    log(f"[small] {name}: T={w.T} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} k={w.topk} "
        f"n_q={w.n_q} bq={w.block_q} {w.dtype}")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    errs = [compare_head(w, gpu, oracle_head(w, 0, h), h) for h in range(w.H_sel)]
    log(f"  max-abs out err {max(errs):.3e}")


def test_exact_ties_lower_index_wins():
    """Integer-valued inputs: many spans tie exactly; fp64 sums are exact on
    both sides, so the lower-index rule must be reproduced bit-exactly."""
    rng = np.random.default_rng(1234)
    w = S(Hq=4, Hkv=2, d=64, T=1200, S=16, topk=11, L=64, needles=0)
    qn = rng.integers(0, 2, size=(1, w.Hq, w.d)).astype(np.float32)
    Kn = rng.integers(0, 2, size=(w.Hkv, w.T, w.d)).astype(np.float32)
    Kn[:, 200:260] = Kn[:, 300:360]           # duplicated spans -> equal scores
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    q, K, V = to_bf(qn), to_bf(Kn), to_bf(Vn)
    gpu = run_library(w, q, K, V)
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    split_groups = 0
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"][0]
        kth = np.sort(sc)[::-1][w.topk - 1]
        above, tied = int((sc > kth).sum()), int((sc == kth).sum())
        log(f"  head {h}: {above} above the k-th score, {tied} tied at it")
        split_groups += above < w.topk < above + tied
        compare_head(w, gpu, ora, h)
    assert split_groups >= 1       # the k-th boundary cuts through a tie group


@pytest.mark.parametrize("T,S_,k", [(40000, 16, 40), (60000, 8, 300), (200000, 4, 600),
                                    (150000, 2, 2000), (200000, 1, 600), (300000, 1, 3000),
                                    (100000, 16, 100), (90000, 12, 64)])
def test_exact_ties_many_candidates(T, S_, k):
    """Binary inputs over thousands of spans, the k-th boundary cutting a tie
    group, through each way the top-k step can go: under 192 candidates
    (pairwise ranks), thousands of candidates (histogram levels down to the
    by-index level), more than 256 candidate groups and more than 2048 groups
    (the generic path over global memory).  Token level (S = 1): the groups
    with one token at or above the bound are taken from the scorer's second
    largest score and the offset of the maximum, the others (two or more, or
    a tied maximum) read token by token.  Spans with k <= 128 over more than
    4096 spans (the last two cases): candidate groups whose third largest score
    is below the bound give their spans from the scorer's top three, the
    others (tied tops) are read, and with more than 192 candidates the cutoff
    and a span bitmap give the output."""
    rng = np.random.default_rng(T + k)
    w = S(Hq=2, Hkv=2, d=64, T=T, S=S_, topk=k, L=64, needles=0)
    qn = rng.integers(0, 2, size=(1, w.Hq, w.d)).astype(np.float32)
    Kn = rng.integers(0, 2, size=(w.Hkv, w.T, w.d)).astype(np.float32)
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    split, crowded = 0, 0
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"][0]
        kth = np.sort(sc)[::-1][w.topk - 1]
        above, tied = int((sc > kth).sum()), int((sc == kth).sum())
        # spans at or above the k-th largest group maximum: a lower bound of
        # the candidates the top-k step ranks
        gmax = np.array([sc[i:i + 32].max() for i in range(0, len(sc), 32)])
        cand = int((sc >= np.sort(gmax)[::-1][min(w.topk, len(gmax)) - 1]).sum())
        log(f"  head {h}: {len(sc)} spans, {above} above the k-th, {tied} tied, >= {cand} candidates")
        split += above < w.topk < above + tied
        crowded += cand > 192
        compare_head(w, gpu, ora, h)
    assert split >= 1 and (crowded >= 1 or T == 40000)


def test_token_level_many_two_candidate_groups():
    """Token level, 3000 groups of 32 tokens holding two equal high tokens each
    (every other token scores 0) and k = 3000: every candidate group has its
    second largest score at the bound, more of them than the list of groups to
    read holds, so the top-k reads every candidate group; the 3000 selected
    are the lowest indices of the 6000 tied tokens."""
    rng = np.random.default_rng(4242)
    w = S(Hq=2, Hkv=2, d=64, T=200000, S=1, topk=3000, L=64, needles=0)
    lo, hi = w.mid
    n_groups = (hi - lo) // 32
    qn = np.ones((1, w.Hq, w.d), np.float32)
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    for h in range(w.Hkv):
        for gi in rng.choice(n_groups, size=3000, replace=False):
            a, b = rng.choice(32, size=2, replace=False)
            Kn[h, lo + gi * 32 + a] = 1.0
            Kn[h, lo + gi * 32 + b] = 1.0
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"][0]
        assert int((sc == sc.max()).sum()) == 6000
        compare_head(w, gpu, ora, h)


def test_token_order_below_fp32_resolution():
    """fp32 inputs whose token scores differ only below fp32 resolution
    (score = level + 2^-30 * noise): the top-k's large path bounds the k-th
    score with group maxima rounded up to fp32, which tie in large numbers;
    the selection must still be the exact fp64 one."""
    rng = np.random.default_rng(2024)
    w = S(dtype="f32", Hq=1, Hkv=1, d=64, T=70000, S=1, topk=3000, L=64, needles=0)
    qn = np.zeros((1, w.Hq, w.d), np.float32)
    qn[0, 0, 0], qn[0, 0, 1] = 1.0, 2.0 ** -30
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    Kn[0, :, 0] = rng.integers(0, 40, size=w.T)
    Kn[0, :, 1] = rng.uniform(-1.0, 1.0, size=w.T)
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    gpu = run_library(w, dev(qn), dev(Kn), dev(Vn))
    ora = oracle_head(w, 0, 0, qn.astype(np.float64), Kn.astype(np.float64), Vn.astype(np.float64))
    sc = ora["sc"][0]
    kth = np.sort(sc)[::-1][w.topk - 1]
    level = np.rint(kth)
    at_level = int((np.abs(sc - level) < 0.5).sum())
    # the boundary falls inside one integer level, decided by the 2^-30 terms
    assert int((sc > level + 0.5).sum()) < w.topk < int((sc > level - 0.5).sum())
    assert np.float32(level + 2.0 ** -31) == np.float32(level)
    log(f"  k-th score {kth!r}: {at_level} tokens share its integer level")
    compare_head(w, gpu, ora, 0)


def test_exact_ties_mfma_blocks():
    """Integer inputs through the MFMA block path: tied spans share identical
    approximate scores and must be resolved by index after exact re-scoring."""
    rng = np.random.default_rng(4321)
    w = S(Hq=8, Hkv=2, d=128, T=3000, n_q=64, block_q=64, S=32, topk=10, L=128, needles=0)
    qn = rng.integers(0, 2, size=(w.n_q, w.Hq, w.d)).astype(np.float32)
    Kn = rng.integers(0, 2, size=(w.Hkv, w.T, w.d)).astype(np.float32)
    # 14 identical spans that outscore the rest: the top-10 boundary cuts the tie
    pattern = rng.integers(1, 3, size=(w.S, w.d)).astype(np.float32)
    for j in rng.choice(80, size=14, replace=False):
        Kn[:, w.G + j * w.S:w.G + (j + 1) * w.S] = pattern
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    ties = 0
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"][0]
        kth = np.sort(sc)[::-1][w.topk - 1]
        above, tied = int((sc > kth).sum()), int((sc == kth).sum())
        ties += above < w.topk < above + tied
        compare_head(w, gpu, ora, h)
    assert ties == w.Hkv


@pytest.mark.parametrize("n_q,T", [(64, 3000), (128, 3000), (64, 140000)])
def test_mfma_blocks_order_below_fp32_resolution(n_q, T):
    """MFMA block scores whose spans differ only below fp32 resolution: 30
    spans score 64 * (256 + 2^-12 * v_j) with distinct v_j = 1 + m_j / 128
    (m_j < 32), so their per-token differences (m * 2^-19) lie below the fp32
    ulp of a token score (2^-15 at 256) and only the fp64 re-scoring of the
    uncertain spans orders them; the top-10 boundary falls among them.  Each span's
    approximate score must stay within its bound eps_j, and the selection must
    be the exact one.  At 140,000 tokens (4,371 spans) the certification ranks
    only the candidate spans near the boundary."""
    rng = np.random.default_rng(777 + n_q + T)
    w = S(Hq=8, Hkv=2, d=128, T=T, n_q=n_q, block_q=64, S=32, topk=10, L=128, needles=0)
    qn = np.zeros((w.n_q, w.Hq, w.d), np.float32)
    qn[:, :, 0] = 1.0                              # q_eff[0] = 4 (four heads per KV head)
    qn[:, :, 1] = 2.0 ** -14                       # q_eff[1] = 2^-12
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    Kn[:, :, 0] = 32.0                             # ordinary spans: about 128 per token
    Kn[:, :, 2:] = rng.standard_normal((w.Hkv, w.T, w.d - 2)) * 2.0 ** -20
    lo, hi = w.mid
    n_full = (hi - lo) // w.S
    for h in range(w.Hkv):
        spans = rng.choice(n_full, size=30, replace=False)
        ms = rng.choice(32, size=30, replace=False)     # neighbours at most 3 apart
        for j, m in zip(spans, ms):
            t0 = lo + j * w.S
            Kn[h, t0:t0 + w.S, 0] = 64.0
            # the span's maximum sits on one token; the others score lower
            Kn[h, t0:t0 + w.S, 1] = 1.0
            Kn[h, t0 + int(rng.integers(w.S)), 1] = 1.0 + m / 128.0
    Kn = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Kn))     # noise rounded to bf16
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    assert np.array_equal(bf(Kn), Kn.astype(np.float64)) and np.array_equal(bf(qn), qn)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"]
        for b in range(w.n_q // w.block_q):
            top = np.sort(sc[b])[::-1]
            gap = top[w.topk - 1] - top[w.topk]
            # the exact gap at the boundary is below one fp32 ulp of a token score
            assert 0 < gap < 64 * 2.0 ** -15, (h, b, gap)
            # and the approximate scores cannot order the candidates
            assert ora["eps"][b].max() > 100 * gap
        compare_head(w, gpu, ora, h)
        log(f"  head {h}: worst |s_hat - s| / eps_j = {ora['eps_used']:.3g}")


@pytest.mark.parametrize("T", [3000, 200000])
def test_per_query_head_order_below_fp32_resolution(T):
    """One selection per query head (scored on MFMA in fp32): 30 spans score
    256 + 2^-16 * v_j with distinct v_j = 1 + m_j / 128, so their differences
    (m * 2^-23) lie below the fp32 ulp of a token score (2^-15 at 256) and only
    the fp64 re-scoring orders them; the top-10 boundary falls among them for
    every query head.  At 200,000 tokens the certification ranks only the
    candidate spans near the boundary."""
    rng = np.random.default_rng(99 + T)
    w = S(Hq=8, Hkv=2, d=128, T=T, S=32, topk=10, L=128, needles=0, per_q_head=True)
    qn = np.zeros((1, w.Hq, w.d), np.float32)
    qn[0, :, 0] = 1.0
    qn[0, :, 1] = 2.0 ** -16
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    Kn[:, :, 0] = 128.0
    Kn[:, :, 2:] = rng.standard_normal((w.Hkv, w.T, w.d - 2)) * 2.0 ** -20
    lo, hi = w.mid
    n_full = (hi - lo) // w.S
    for h in range(w.Hkv):
        for j, m in zip(rng.choice(n_full, size=30, replace=False),
                        rng.choice(32, size=30, replace=False)):
            t0 = lo + j * w.S
            Kn[h, t0:t0 + w.S, 0] = 256.0
            Kn[h, t0:t0 + w.S, 1] = 1.0
            Kn[h, t0 + int(rng.integers(w.S)), 1] = 1.0 + m / 128.0
    Kn = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Kn))
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    for u in range(w.H_sel):
        hk = u // w.g
        ora = oracle_head(w, 0, u, q64, K64[hk:hk + 1], V64[hk:hk + 1])
        top = np.sort(ora["sc"][0])[::-1]
        gap = top[w.topk - 1] - top[w.topk]
        assert 0 < gap < 2.0 ** -15 and ora["eps"][0].max() > 100 * gap, (u, gap)
        compare_head(w, gpu, ora, u)


def test_mfma_blocks_massive_ties_past_4096_spans():
    """Beyond 4096 spans, with every span but a few scoring exactly alike
    (integer keys repeating one pattern): the candidates near the k-th score
    would be nearly every span, so the pairs take the exact fallback (fp64
    scores on the VALU, then the ordinary top-k); the 20 raised spans and the
    30 lowest indices of the tie must be selected."""
    rng = np.random.default_rng(5150)
    w = S(Hq=4, Hkv=2, d=128, T=140000, n_q=64, block_q=64, S=32, topk=50, L=128, needles=0)
    assert w.n_spans > 4096
    qn = rng.integers(0, 2, size=(w.n_q, w.Hq, w.d)).astype(np.float32)
    pattern = rng.integers(0, 3, size=(w.S, w.d)).astype(np.float32)
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    lo, hi = w.mid
    n_full = (hi - lo) // w.S
    Kn[:, lo:lo + n_full * w.S] = np.tile(pattern, (n_full, 1))[None]
    for h in range(w.Hkv):
        for j in rng.choice(w.n_spans - 1, size=20, replace=False):
            Kn[h, lo + j * w.S:lo + (j + 1) * w.S] = pattern + 1.0
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64, K64[h:h + 1], V64[h:h + 1])
        sc = ora["sc"][0]
        kth = np.sort(sc)[::-1][w.topk - 1]
        assert int((sc > kth).sum()) == 20 and int((sc == kth).sum()) > 4096
        compare_head(w, gpu, ora, h)


def test_per_query_head_massive_ties_past_4096_spans():
    """One selection per query head, beyond 4096 spans, every span but 20 per
    KV head scoring exactly alike: the candidate spans near the k-th score
    would be nearly all of them, so every pair takes the exact fallback (fp64
    scores on the VALU, then the ordinary top-k); the raised spans and the
    lowest indices of the tie must be selected for each query head."""
    rng = np.random.default_rng(5151)
    w = S(Hq=8, Hkv=2, d=128, T=140000, S=32, topk=50, L=128, needles=0, per_q_head=True)
    assert w.n_spans > 4096
    qn = rng.integers(0, 2, size=(w.n_q, w.Hq, w.d)).astype(np.float32)
    qn[..., 0] = 1.0                            # every query head sums above zero
    pattern = rng.integers(0, 3, size=(w.S, w.d)).astype(np.float32)
    Kn = np.zeros((w.Hkv, w.T, w.d), np.float32)
    lo, hi = w.mid
    n_full = (hi - lo) // w.S
    Kn[:, lo:lo + n_full * w.S] = np.tile(pattern, (n_full, 1))[None]
    for h in range(w.Hkv):
        for j in rng.choice(w.n_spans - 1, size=20, replace=False):
            Kn[h, lo + j * w.S:lo + (j + 1) * w.S] = pattern + 1.0
    Vn = rng.standard_normal((w.Hkv, w.T, w.d)).astype(np.float32)
    to_bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    bf = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    gpu = run_library(w, to_bf(qn), to_bf(Kn), to_bf(Vn))
    q64, K64, V64 = bf(qn), bf(Kn), bf(Vn)
    for h in range(w.Hq):
        hp = h // w.g
        ora = oracle_head(w, 0, h, q64, K64[hp:hp + 1], V64[hp:hp + 1])
        sc = ora["sc"][0]
        kth = np.sort(sc)[::-1][w.topk - 1]
        assert int((sc > kth).sum()) == 20 and int((sc == kth).sum()) > 4096
        compare_head(w, gpu, ora, h)


def test_deterministic():
    w = SMALL["bf16_many_heads"]
    q, K, V = device_inputs(w)
    a = run_library(w, q, K, V, components=False)
    b = run_library(w, q, K, V, components=False)
    assert np.array_equal(a["out_step"], b["out_step"])
    assert np.array_equal(a["sel_step"], b["sel_step"])


def test_reused_workspace_two_lengths():
    """Decode steps and score-selects at two context lengths with the same
    heads share one workspace, so every call starts from what the one before
    left in it: each must give every span score (the caller's array starts as
    NaN) and the selection the oracle gives, and a repeated step the same
    output."""
    import top_kv_cache_amd as rea
    shapes = {"A": S(Hq=8, Hkv=2, d=128, T=300_000, S=32, topk=40, L=256, needles=2,
                     kv_scaled=True),
              "B": S(Hq=8, Hkv=2, d=128, T=120_000, S=32, topk=40, L=256, needles=2, seed=11)}
    runs = {}
    for key, w in shapes.items():
        q, K, V = device_inputs(w)
        st = rea.Step(q, K, V, w.G, w.S, w.topk, w.L, w.block_q, rope_theta=w.rope_theta)
        q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
        runs[key] = (w, st, [oracle_head(w, 0, h, q64) for h in range(w.Hkv)])
    nbytes = max(max(st.sizes.ws_decode_step, st.sizes.ws_score_select)
                 for _, st, _ in runs.values())
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:]
    first_out = {}
    for i, key in enumerate(["A", "A", "B", "B", "A", "B"]):
        w, st, ora = runs[key]
        log(f"[reuse] call {i}: T={w.T} ({'score_select' if i % 2 else 'decode_step'})")
        if i % 2:
            sel, nsel, sc = st.score_select(span_scores=True, ws=ws)
            sc = sc.cpu().numpy()
            for h in range(w.Hkv):
                ref = ora[h]["sc"][0]
                assert not np.isnan(sc[0, h]).any(), ("unwritten span scores", key, h)
                assert np.abs(sc[0, h] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
        else:
            nb, cap = st.sizes.n_blocks, w.sel_cap
            sel = torch.full((nb, w.Hkv, cap), -7, dtype=torch.int32, device="cuda")
            nsel = torch.empty((nb, w.Hkv), dtype=torch.int32, device="cuda")
            out = st.decode_step(sel=sel, nsel=nsel, ws=ws).cpu().numpy()
            if key in first_out:
                assert np.array_equal(out, first_out[key])
            first_out.setdefault(key, out)
        sel, nsel = sel.cpu().numpy(), nsel.cpu().numpy()
        for h in range(w.Hkv):
            exp = ora[h]["sel"][0]
            assert int(nsel[0, h]) == len(exp)
            assert sel[0, h, :len(exp)].tolist() == exp, (i, key, h)


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_one_layer(cfg):
    w = synth.config(cfg)
    log(f"[config {cfg}] {w.name}")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    errs = []
    for h in range(w.Hkv):
        ora = oracle_head(w, 0, h, q64)
        errs.append(compare_head(w, gpu, ora, h))
        needles = [j for (hh, j) in w.needle_spans(0) if hh == h]
        assert set(needles) <= set(ora["sel"][0])
    log(f"  max-abs out err {max(errs):.3e} (tolerance {TOL[w.dtype]})")


VARIANTS = {
    # the 8B decode at 131072 tokens with one selection per query head
    "per_q_head": dict(per_q_head=True),
    # token-level selection: spans of one token, the same 3840-token budget
    "token_level": dict(S=1, topk=3840),
    # the 120 best tokens, each widened to 32 tokens
    "token_segments": dict(token_segments=True),
    # the pages' own LLaMA3-8B-8K tuple: 127 spans, window exactly 8192
    "pages_k127": dict(topk=127),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_config2_variant(variant):
    w = dataclasses.replace(synth.config(2), **VARIANTS[variant])
    w.name = f"{w.name}-{variant}"
    log(f"[variant] {w.name}: S={w.S} k={w.topk} per_q_head={w.per_q_head} "
        f"token_segments={w.token_segments}")
    q, K, V = device_inputs(w)
    gpu = run_library(w, q, K, V)
    del K, V
    torch.cuda.empty_cache()
    q64 = synth.to_f32(w.q(0), w.dtype).astype(np.float64)
    errs = []
    for h in range(w.H_sel):
        ora = oracle_head(w, 0, h, q64)
        errs.append(compare_head(w, gpu, ora, h))
    log(f"  max-abs out err {max(errs):.3e} (tolerance {TOL[w.dtype]})")
