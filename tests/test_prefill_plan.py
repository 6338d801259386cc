"""Chunked-prefill plan on the host: the chunks rea_prefill_plan reports match
the rule its header states (first chunk min(T, G+L) rounded down to a multiple
of block_q, then chunks of `chunk` tokens; a chunk whose length is not a
multiple of block_q is cut into equal blocks of the largest divisor not above
block_q), and bad arguments are rejected without a GPU."""
import ctypes

import pytest

import top_kv_cache_amd as rea

FAKE = 0x10000          # an aligned non-null address; nothing is launched


def expected_plan(T, G, L, bq, chunk):
    out, pos = [], 0
    first = min(T, G + L)
    first -= first % bq
    if first > 0:
        out.append((0, first, bq))
        pos = first
    while pos < T:
        n = min(chunk, T - pos)
        b = max(x for x in range(1, min(bq, n) + 1) if n % x == 0)
        out.append((pos, n, b))
        pos += n
    return out


def make(T, G, S, k, L, bq, dtype=rea.REA_BF16, Hq=8, Hkv=2, d=128):
    p = rea.problem(FAKE, FAKE, FAKE, dtype=dtype, n_q=T, Hq=Hq, Hkv=Hkv, d=d, T=T,
                    stride_head=T * d, stride_tok=d)
    return p, rea.params(G, S, k, L, bq)


@pytest.mark.parametrize("T,G,S,k,L,bq,chunk", [
    (3000, 8, 16, 12, 256, 64, 128),        # last chunk 56 tokens: blocks of 56
    (700, 4, 8, 6, 64, 16, 32),
    (135168, 32, 32, 120, 4096, 64, 512),   # a 132K-token prompt at the pages' settings
    (200, 32, 32, 120, 4096, 64, 512),      # shorter than G + L: one chunk, no middle
    (4100, 32, 32, 120, 4096, 64, 512),     # G + L = 4128 > T: first 4096, then 4
    (1031, 4, 16, 8, 128, 32, 96),          # 1031 - 128 = 903 = 9 x 96 + 39: blocks of 13
])
def test_plan_follows_the_stated_rule(T, G, S, k, L, bq, chunk):
    p, a = make(T, G, S, k, L, bq)
    plan, ws = rea.prefill_plan(p, a, chunk)
    assert plan == expected_plan(T, G, L, bq, chunk)
    # blocks are numbered in plan order for rea_prefill's selection outputs
    plan4, n_blocks, ws4 = rea.prefill_plan(p, a, chunk, with_blocks=True)
    assert [c[:3] for c in plan4] == plan and ws4 == ws
    first = 0
    for (s0, n, b, fb) in plan4:
        assert fb == first
        first += n // b
    assert n_blocks == first
    # contiguous cover of the prompt, each block size dividing its chunk
    assert plan[0][0] == 0 and sum(n for _, n, _ in plan) == T
    for (s0, n0, _), (s1, _, _) in zip(plan, plan[1:]):
        assert s1 == s0 + n0
    assert all(n % b == 0 and 1 <= b <= bq for _, n, b in plan)
    # the workspace covers every chunk's decode step
    for s0, n, b in plan:
        pc = rea.problem(FAKE, FAKE, FAKE, dtype=p.dtype, n_q=n, Hq=p.n_q_heads,
                         Hkv=p.n_kv_heads, d=p.head_dim, T=s0 + n, stride_head=p.kv_stride_head,
                         stride_tok=p.kv_stride_tok)
        ac = rea.params(G, S, k, L, b)
        assert rea.query_sizes(pc, ac).ws_decode_step <= ws


def status_of(p, a, chunk):
    n, ws = ctypes.c_int32(), ctypes.c_size_t()
    return rea.lib().rea_prefill_plan(ctypes.byref(p), ctypes.byref(a), chunk, None, 0,
                                      ctypes.byref(n), None, ctypes.byref(ws))


def test_plan_rejects_bad_arguments():
    EINVAL = rea.STATUS.index("REA_EINVAL")
    p, a = make(3000, 8, 16, 12, 256, 64)
    assert status_of(p, a, 0) == EINVAL            # empty chunk
    assert status_of(p, a, 96) == EINVAL           # not a multiple of block_q
    assert status_of(p, a, 512) == EINVAL          # longer than L
    q = rea.problem(FAKE, FAKE, FAKE, dtype=rea.REA_BF16, n_q=1, Hq=8, Hkv=2, d=128, T=3000,
                    stride_head=3000 * 128, stride_tok=128)
    assert status_of(q, a, 128) == EINVAL          # not every prompt token is a query
    assert "n_q" in rea.lib().rea_last_error().decode()
    L = rea.lib()
    assert L.rea_prefill(ctypes.byref(p), ctypes.byref(a), 128, None, None, None, None, 0,
                         None) == EINVAL           # out is NULL
    assert L.rea_prefill(ctypes.byref(p), ctypes.byref(a), 128, FAKE, FAKE, None, None, 0,
                         None) == EINVAL           # sel without n_sel
    assert L.rea_prefill(ctypes.byref(p), ctypes.byref(a), 128, FAKE, FAKE + 2, FAKE, None, 0,
                         None) == rea.STATUS.index("REA_EALIGN")
