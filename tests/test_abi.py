"""C-ABI contract on the host: the library loads, exports every declared entry
point, reports sizes, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import top_kv_cache_amd as rea
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # an aligned non-null address; nothing is launched


def declared_symbols(header="rea.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rea_[a-z_]+)\s*\(", text)))


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["rea.h", "rea_probe.h"]


def test_exports_the_probe():
    L = rea.lib()
    syms = declared_symbols("rea_probe.h")
    assert syms == sorted(rea.PROBE_ENTRY_POINTS)
    for s in syms:
        assert hasattr(L, s), s
    # invalid arguments are refused before any launch
    assert L.rea_probe_stream_read(None, 1024, 2, 8, FAKE, None) == 1
    assert L.rea_probe_stream_read(FAKE, 1000, 2, 8, FAKE, None) == 1
    assert L.rea_probe_stream_read(FAKE, 1024, 2, 5, FAKE, None) == 1


def test_exports_every_declared_symbol():
    L = rea.lib()
    syms = declared_symbols()
    # the boundary's calls: score/select, gather+RoPE, window attention, the
    # fused step and the workspace size
    assert set(syms) >= {"rea_score_select", "rea_gather_rope", "rea_window_attend",
                         "rea_decode_step", "rea_workspace_bytes", "rea_status_string",
                         "rea_last_error"}
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(rea.ENTRY_POINTS) == syms
    assert L.rea_abi_version() == 4
    for i, name in enumerate(rea.STATUS):
        assert L.rea_status_string(i).decode() == name


def good(dtype=rea.REA_BF16, n_q=1, Hq=32, Hkv=8, d=128, T=131072):
    p = rea.problem(FAKE, FAKE, FAKE, dtype=dtype, n_q=n_q, Hq=Hq, Hkv=Hkv, d=d, T=T,
                    stride_head=T * d, stride_tok=d)
    a = rea.params(32, 32, 120, 4096, 1)
    return p, a


def sizes_status(p, a):
    s = rea.Sizes()
    return rea.lib().rea_query_sizes(ctypes.byref(p), ctypes.byref(a), ctypes.byref(s)), s


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_sizes_match_workloads(cfg):
    w = synth.config(cfg)
    p = rea.problem(FAKE, FAKE, FAKE, dtype=rea.REA_BF16 if w.dtype == "bf16" else rea.REA_F32,
                    n_q=w.n_q, Hq=w.Hq, Hkv=w.Hkv, d=w.d, T=w.T, stride_head=w.T * w.d,
                    stride_tok=w.d)
    a = rea.params(w.G, w.S, w.topk, w.L, w.block_q)
    st, s = sizes_status(p, a)
    assert st == 0, rea.lib().rea_last_error()
    assert s.n_spans == w.n_spans
    assert s.k_sel == min(w.topk, w.n_spans)
    assert s.W_cap == w.W_cap
    assert s.n_blocks == w.n_q // w.block_q
    assert s.ws_decode_step >= s.ws_score_select > 0


def mutate(**kw):
    p, a = good()
    for k, v in kw.items():
        if hasattr(p, k):
            setattr(p, k, v)
        else:
            setattr(a, k, v)
    return p, a


@pytest.mark.parametrize("kw,expect", [
    (dict(struct_size=12), rea.STATUS.index("REA_EINVAL")),
    (dict(q=None), rea.STATUS.index("REA_EINVAL")),
    (dict(k=None), rea.STATUS.index("REA_EINVAL")),
    (dict(S=0), rea.STATUS.index("REA_EINVAL")),
    (dict(topk=-1), rea.STATUS.index("REA_EINVAL")),
    (dict(G=-1), rea.STATUS.index("REA_EINVAL")),
    (dict(L=-5), rea.STATUS.index("REA_EINVAL")),
    (dict(block_q=0), rea.STATUS.index("REA_EINVAL")),
    (dict(select_flags=4), rea.STATUS.index("REA_EINVAL")),
    (dict(rope_theta=0.0), rea.STATUS.index("REA_EINVAL")),
    (dict(rope_theta=float("inf")), rea.STATUS.index("REA_EINVAL")),
    (dict(softmax_scale=float("nan")), rea.STATUS.index("REA_EINVAL")),
    (dict(dtype=7), rea.STATUS.index("REA_EDTYPE")),
    (dict(n_q_heads=30), rea.STATUS.index("REA_ESHAPE")),
    (dict(n_kv_heads=0), rea.STATUS.index("REA_ESHAPE")),
    (dict(n_q=0), rea.STATUS.index("REA_ESHAPE")),
    (dict(n_q=4, block_q=3), rea.STATUS.index("REA_ESHAPE")),
    (dict(T=0), rea.STATUS.index("REA_ESHAPE")),
    (dict(T=1 << 31), rea.STATUS.index("REA_ESHAPE")),
    (dict(kv_stride_tok=64), rea.STATUS.index("REA_ESHAPE")),
    (dict(kv_stride_head=128), rea.STATUS.index("REA_ESHAPE")),
    (dict(n_q=4097, block_q=1), rea.STATUS.index("REA_ESHAPE")),   # queries beyond the local region
    (dict(head_dim=96), rea.STATUS.index("REA_EUNSUPPORTED")),
    (dict(k=FAKE + 8), rea.STATUS.index("REA_EALIGN")),
    (dict(kv_stride_tok=132), rea.STATUS.index("REA_EALIGN")),
    (dict(n_q=128, block_q=128), rea.STATUS.index("REA_EUNSUPPORTED")),
])
def test_invalid_arguments(kw, expect):
    p, a = mutate(**kw)
    if "head_dim" in kw:
        p.kv_stride_tok, p.kv_stride_head = kw["head_dim"], p.T * kw["head_dim"]
    if kw.get("kv_stride_tok") == 132:      # misaligned rows, no overlap
        p.kv_stride_head = p.T * 132
    st, _ = sizes_status(p, a)
    assert st == expect, (rea.STATUS[st], rea.lib().rea_last_error())
    assert rea.lib().rea_last_error().decode() != ""
    # the entry points run the same validation before any HIP call
    L = rea.lib()
    st2 = L.rea_score_select(ctypes.byref(p), ctypes.byref(a), FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st2 == expect
    st3 = L.rea_decode_step(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, FAKE, 1 << 40,
                            None)
    assert st3 == expect
    st4 = L.rea_decode_step_timed(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, FAKE,
                                  1 << 40, None, None)
    assert st4 == expect
    assert L.rea_workspace_bytes(ctypes.byref(p), ctypes.byref(a)) == rea.WORKSPACE_INVALID


def test_no_middle_allows_many_queries():
    # T <= G + L: every query may be anywhere (plain causal attention)
    p, a = good(n_q=64, T=1000)
    a.block_q = 64
    st, s = sizes_status(p, a)
    assert st == 0 and s.n_spans == 0 and s.W_cap == 1000 and s.k_sel == 0


def test_entry_point_argument_errors():
    L = rea.lib()
    p, a = good()
    _, s = sizes_status(p, a)
    E = rea.STATUS.index
    # workspace too small / misaligned
    assert L.rea_score_select(ctypes.byref(p), ctypes.byref(a), FAKE, FAKE, None, FAKE,
                              s.ws_score_select - 1, None) == E("REA_EWORKSPACE")
    assert L.rea_score_select(ctypes.byref(p), ctypes.byref(a), FAKE, FAKE, None, FAKE + 16,
                              s.ws_score_select, None) == E("REA_EALIGN")
    assert L.rea_decode_step(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, FAKE,
                             s.ws_decode_step - 1, None) == E("REA_EWORKSPACE")
    # null outputs
    assert L.rea_score_select(ctypes.byref(p), ctypes.byref(a), None, FAKE, None, FAKE,
                              s.ws_score_select, None) == E("REA_EINVAL")
    assert L.rea_decode_step(ctypes.byref(p), ctypes.byref(a), None, None, None, FAKE,
                             s.ws_decode_step, None) == E("REA_EINVAL")
    # window capacity too small
    assert L.rea_gather_rope(ctypes.byref(p), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, int(s.W_cap) - 1, None) == E("REA_ESHAPE")
    assert L.rea_window_attend(ctypes.byref(p), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE,
                               int(s.W_cap), FAKE, FAKE, s.ws_window_attend - 1,
                               None) == E("REA_EWORKSPACE")


def test_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = rea.lib()
    p, a = good()
    _, s = sizes_status(p, a)
    st = L.rea_decode_step(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, FAKE,
                           s.ws_decode_step, None)
    assert st == rea.STATUS.index("REA_ENODEVICE"), L.rea_last_error()
    st = L.rea_decode_step_timed(ctypes.byref(p), ctypes.byref(a), FAKE, None, None, FAKE,
                                 s.ws_decode_step, None, None)
    assert st == rea.STATUS.index("REA_ENODEVICE"), L.rea_last_error()


def test_sizes_per_query_head_selection():
    p, a = good()
    st, s = sizes_status(p, a)
    assert st == 0 and s.n_sel_heads == 8
    a.select_flags = rea.REA_SELECT_PER_Q_HEAD
    st, s2 = sizes_status(p, a)
    assert st == 0, rea.lib().rea_last_error()
    assert s2.n_sel_heads == 32 and s2.n_spans == s.n_spans and s2.W_cap == s.W_cap
    assert s2.ws_decode_step > s.ws_decode_step      # four times the span scores
    # token level: spans of one token
    a.S, a.topk = 1, 3840
    st, s3 = sizes_status(p, a)
    assert st == 0 and s3.n_spans == 131072 - 32 - 4096 and s3.W_cap == 32 + 3840 + 4096


def test_batched_decode_workspace_and_errors():
    L = rea.lib()
    E = rea.STATUS.index
    p, a = good()
    ws = ctypes.c_size_t()
    assert L.rea_decode_batch_workspace(ctypes.byref(p), ctypes.byref(a), 4, ctypes.byref(ws)) == 0
    ws4 = ws.value
    assert L.rea_decode_batch_workspace(ctypes.byref(p), ctypes.byref(a), 1, ctypes.byref(ws)) == 0
    ws1 = ws.value
    _, s = sizes_status(p, a)
    assert ws1 == s.ws_decode_step and ws4 > 3 * ws1
    assert L.rea_decode_batch_workspace(ctypes.byref(p), ctypes.byref(a), 0,
                                        ctypes.byref(ws)) == E("REA_EINVAL")
    stride = p.n_kv_heads * p.kv_stride_head

    def call(pp=p, aa=a, batch=4, lens=FAKE, kvs=stride, out=FAKE, wsb=ws4):
        return L.rea_decode_batch(ctypes.byref(pp), ctypes.byref(aa), batch, lens, kvs, out,
                                  None, None, FAKE, wsb, None)

    assert call(lens=None) == E("REA_EINVAL")
    assert call(lens=FAKE + 4) == E("REA_EALIGN")
    assert call(kvs=stride - 8) == E("REA_ESHAPE")
    assert call(kvs=stride + 4) == E("REA_EALIGN")
    assert call(out=None) == E("REA_EINVAL")
    assert call(wsb=ws4 - 1) == E("REA_EWORKSPACE")
    p2, a2 = good(n_q=2)
    a2.block_q = 2
    assert call(pp=p2, aa=a2) == E("REA_EUNSUPPORTED")
    # 16 query heads per KV head: fp32 has only the VALU attention (at most 8)
    p3, a3 = good(dtype=rea.REA_F32, Hq=64, Hkv=4)
    assert call(pp=p3, aa=a3, kvs=p3.n_kv_heads * p3.kv_stride_head) == E("REA_EUNSUPPORTED")
    a4 = rea.params(32, 32, 120, 0, 1)
    assert call(aa=a4) == E("REA_ESHAPE")   # L = 0: the query token would not be local
    p5, a5 = good(T=32)                     # T <= G + L passes the one-sequence check
    a5.L = 0
    assert call(pp=p5, aa=a5, kvs=p5.n_kv_heads * p5.kv_stride_head) == E("REA_EINVAL")
    import torch
    if not torch.cuda.is_available():
        assert call() == E("REA_ENODEVICE")


def test_sizes_token_segments():
    p, a = good()
    a.select_flags = rea.REA_SELECT_TOKEN_SEGMENTS
    st, s = sizes_status(p, a)
    assert st == 0, rea.lib().rea_last_error()
    n_mid = 131072 - 32 - 4096
    assert s.n_spans == n_mid and s.k_sel == 120 * 32 and s.W_cap == 32 + 120 * 32 + 4096
    a.select_flags = rea.REA_SELECT_TOKEN_SEGMENTS | rea.REA_SELECT_PER_Q_HEAD
    st, s2 = sizes_status(p, a)
    assert st == 0 and s2.n_sel_heads == 32 and s2.ws_decode_step > s.ws_decode_step


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workspace_bytes_covers_every_entry_point(cfg):
    """rea_workspace_bytes is the largest of the three workspaces rea_query_sizes
    reports, for the default selection and each variant."""
    w = synth.config(cfg)
    for extra in (dict(), dict(per_q_head=True), dict(token_segments=True)):
        p = rea.problem(FAKE, FAKE, FAKE, dtype=rea.REA_BF16 if w.dtype == "bf16" else rea.REA_F32,
                        n_q=w.n_q, Hq=w.Hq, Hkv=w.Hkv, d=w.d, T=w.T, stride_head=w.T * w.d,
                        stride_tok=w.d)
        a = rea.params(w.G, w.S, w.topk, w.L, w.block_q, **extra)
        s = rea.query_sizes(p, a)
        n = rea.workspace_bytes(p, a)
        assert n == max(s.ws_score_select, s.ws_window_attend, s.ws_decode_step) > 0


def test_noalloc_validates_on_the_host():
    """rea_decode_step_noalloc runs rea_decode_step's checks before any HIP
    call, and rejects steps whose workspace exceeds its fixed scratch array."""
    L = rea.lib()
    E = rea.STATUS.index
    p, a = good()
    assert rea.query_sizes(p, a).ws_decode_step <= rea.NOALLOC_SCRATCH_BYTES
    assert L.rea_decode_step_noalloc(ctypes.byref(p), ctypes.byref(a), None, None, None,
                                     None) == E("REA_EINVAL")
    assert L.rea_decode_step_noalloc(ctypes.byref(p), ctypes.byref(a), FAKE + 4, None, None,
                                     None) == E("REA_EALIGN")
    bad, a2 = mutate(S=0)
    assert L.rea_decode_step_noalloc(ctypes.byref(bad), ctypes.byref(a2), FAKE, None, None,
                                     None) == E("REA_EINVAL")
    big = rea.params(32, 1, 3840, 4096, 1)             # token level at 131072: ~9.6 MB, fits
    assert rea.query_sizes(p, big).ws_decode_step <= rea.NOALLOC_SCRATCH_BYTES
    p1m, _ = good(T=1 << 20)                           # token level at 1M: ~70 MB, does not
    assert rea.query_sizes(p1m, big).ws_decode_step > rea.NOALLOC_SCRATCH_BYTES
    assert L.rea_decode_step_noalloc(ctypes.byref(p1m), ctypes.byref(big), FAKE, None, None,
                                     None) == E("REA_EWORKSPACE")
    assert "scratch" in L.rea_last_error().decode()
    import torch
    if not torch.cuda.is_available():
        assert L.rea_decode_step_noalloc(ctypes.byref(p), ctypes.byref(a), FAKE, None, None,
                                         None) == E("REA_ENODEVICE")
