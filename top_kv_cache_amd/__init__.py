"""Python binding of librea.so (the ReAttention hot path on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``).  The library must be built
(``python -m top_kv_cache_amd._build``); importing the package never falls back
to any other implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librea.so")

REA_BF16, REA_F32 = 0, 1
REA_SELECT_PER_Q_HEAD, REA_SELECT_TOKEN_SEGMENTS = 1, 2
STATUS = ["REA_OK", "REA_EINVAL", "REA_ESHAPE", "REA_EDTYPE", "REA_EALIGN",
          "REA_EWORKSPACE", "REA_ENODEVICE", "REA_ELAUNCH", "REA_EUNSUPPORTED"]
ENTRY_POINTS = ["rea_abi_version", "rea_status_string", "rea_last_error", "rea_query_sizes",
                "rea_workspace_bytes", "rea_score_select", "rea_gather_rope",
                "rea_window_attend", "rea_decode_step", "rea_decode_step_timed",
                "rea_prefill_plan", "rea_prefill", "rea_decode_batch_workspace",
                "rea_decode_batch", "rea_decode_step_noalloc"]
# measurement aid (include/rea_probe.h), not part of the method
PROBE_ENTRY_POINTS = ["rea_probe_stream_read", "rea_probe_cu_count"]
ABI_VERSION = 4
NOALLOC_SCRATCH_BYTES = 16 << 20          # REA_NOALLOC_SCRATCH_BYTES
WORKSPACE_INVALID = ctypes.c_size_t(-1).value     # rea_workspace_bytes on invalid arguments


class Problem(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("T", ctypes.c_int64), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("kv_stride_head", ctypes.c_int64),
                ("kv_stride_tok", ctypes.c_int64)]


class Params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("G", ctypes.c_int32), ("S", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("L", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("select_flags", ctypes.c_int32)]


class Sizes(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int64), ("n_spans", ctypes.c_int64),
                ("k_sel", ctypes.c_int64), ("W_cap", ctypes.c_int64),
                ("ws_score_select", ctypes.c_size_t), ("ws_window_attend", ctypes.c_size_t),
                ("ws_decode_step", ctypes.c_size_t), ("n_sel_heads", ctypes.c_int64)]


class Timing(ctypes.Structure):
    _fields_ = [("score_begin", ctypes.c_void_p), ("score_end", ctypes.c_void_p)]


class Chunk(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("n_q", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("first_block", ctypes.c_int64)]


class ReaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{name}: {detail}")


_lib = None


def lib():
    """Load librea.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python -m top_kv_cache_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    P, A = ctypes.POINTER(Problem), ctypes.POINTER(Params)
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    L.rea_abi_version.restype = ctypes.c_int
    L.rea_status_string.restype = ctypes.c_char_p
    L.rea_status_string.argtypes = [ctypes.c_int]
    L.rea_last_error.restype = ctypes.c_char_p
    L.rea_query_sizes.restype = ctypes.c_int
    L.rea_query_sizes.argtypes = [P, A, ctypes.POINTER(Sizes)]
    L.rea_workspace_bytes.restype = ctypes.c_size_t
    L.rea_workspace_bytes.argtypes = [P, A]
    L.rea_score_select.restype = ctypes.c_int
    L.rea_score_select.argtypes = [P, A, i32p, i32p, vp, vp, ctypes.c_size_t, vp]
    L.rea_gather_rope.restype = ctypes.c_int
    L.rea_gather_rope.argtypes = [P, A, i32p, i32p, vp, vp, vp, i32p, ctypes.c_int32, vp]
    L.rea_window_attend.restype = ctypes.c_int
    L.rea_window_attend.argtypes = [P, A, vp, vp, vp, i32p, ctypes.c_int32, vp, vp,
                                    ctypes.c_size_t, vp]
    L.rea_decode_step.restype = ctypes.c_int
    L.rea_decode_step.argtypes = [P, A, vp, i32p, i32p, vp, ctypes.c_size_t, vp]
    L.rea_decode_step_timed.restype = ctypes.c_int
    L.rea_decode_step_timed.argtypes = [P, A, vp, i32p, i32p, vp, ctypes.c_size_t, vp,
                                        ctypes.POINTER(Timing)]
    L.rea_decode_step_noalloc.restype = ctypes.c_int
    L.rea_decode_step_noalloc.argtypes = [P, A, vp, i32p, i32p, vp]
    L.rea_prefill_plan.restype = ctypes.c_int
    L.rea_prefill_plan.argtypes = [P, A, ctypes.c_int32, ctypes.POINTER(Chunk), ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(ctypes.c_size_t)]
    L.rea_prefill.restype = ctypes.c_int
    L.rea_prefill.argtypes = [P, A, ctypes.c_int32, vp, i32p, i32p, vp, ctypes.c_size_t, vp]
    L.rea_decode_batch_workspace.restype = ctypes.c_int
    L.rea_decode_batch_workspace.argtypes = [P, A, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    L.rea_decode_batch.restype = ctypes.c_int
    L.rea_decode_batch.argtypes = [P, A, ctypes.c_int32, vp, ctypes.c_int64, vp, i32p, i32p, vp,
                                   ctypes.c_size_t, vp]
    L.rea_probe_stream_read.restype = ctypes.c_int
    L.rea_probe_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp, vp]
    L.rea_probe_cu_count.restype = ctypes.c_int
    if L.rea_abi_version() != ABI_VERSION:
        raise ImportError(f"librea.so ABI version {L.rea_abi_version()} != {ABI_VERSION}: rebuild it")
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise ReaError(status, lib().rea_last_error().decode())


# ---------------------------------------------------------------------------
# struct builders (plain values; pointers as ints)
# ---------------------------------------------------------------------------
def problem(q_ptr, k_ptr, v_ptr, *, dtype, n_q, Hq, Hkv, d, T, stride_head, stride_tok) -> Problem:
    return Problem(ctypes.sizeof(Problem), dtype, n_q, Hq, Hkv, d, T, q_ptr, k_ptr, v_ptr,
                   stride_head, stride_tok)


def params(G, S, topk, L, block_q=1, rope_theta=500000.0, softmax_scale=0.0,
           per_q_head=False, token_segments=False) -> Params:
    flags = (REA_SELECT_PER_Q_HEAD if per_q_head else 0) | \
        (REA_SELECT_TOKEN_SEGMENTS if token_segments else 0)
    return Params(ctypes.sizeof(Params), G, S, topk, L, block_q, rope_theta, softmax_scale, flags)


def prefill_plan(p: Problem, a: Params, chunk: int, with_blocks: bool = False):
    """(list of (start, n_q, block_q), workspace bytes) of a chunked prefill;
    with_blocks: (list of (start, n_q, block_q, first_block), total blocks,
    workspace bytes).  Host-only (no GPU needed)."""
    n, nb, ws = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_size_t()
    _check(lib().rea_prefill_plan(ctypes.byref(p), ctypes.byref(a), chunk, None, 0,
                                  ctypes.byref(n), ctypes.byref(nb), ctypes.byref(ws)))
    arr = (Chunk * max(n.value, 1))()
    _check(lib().rea_prefill_plan(ctypes.byref(p), ctypes.byref(a), chunk, arr, n.value,
                                  ctypes.byref(n), ctypes.byref(nb), ctypes.byref(ws)))
    if with_blocks:
        return ([(c.start, c.n_q, c.block_q, c.first_block) for c in arr[:n.value]], nb.value,
                ws.value)
    return [(c.start, c.n_q, c.block_q) for c in arr[:n.value]], ws.value


def workspace_bytes(p: Problem, a: Params) -> int:
    """rea_workspace_bytes (raises on invalid arguments).  Host-only."""
    n = lib().rea_workspace_bytes(ctypes.byref(p), ctypes.byref(a))
    if n == WORKSPACE_INVALID:
        raise ReaError(1, lib().rea_last_error().decode())
    return n


def query_sizes(p: Problem, a: Params) -> Sizes:
    s = Sizes()
    _check(lib().rea_query_sizes(ctypes.byref(p), ctypes.byref(a), ctypes.byref(s)))
    return s


# ---------------------------------------------------------------------------
# torch front end
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def problem_from_tensors(q, k, v, T=None) -> Problem:
    """q [n_q][Hq][d] contiguous; k, v [Hkv][T_cap][d] with unit channel stride."""
    torch = _torch()
    if q.dtype == torch.bfloat16:
        dt = REA_BF16
    elif q.dtype == torch.float32:
        dt = REA_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k.stride() != v.stride() or k.shape != v.shape or k.stride(2) != 1:
        raise ValueError("k and v must share shape and strides, channel stride 1")
    n_q, Hq, d = q.shape
    Hkv, Tcap, _ = k.shape
    return problem(q.data_ptr(), k.data_ptr(), v.data_ptr(), dtype=dt, n_q=n_q, Hq=Hq, Hkv=Hkv,
                   d=d, T=Tcap if T is None else T, stride_head=k.stride(0),
                   stride_tok=k.stride(1))


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ws(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)


def _aligned(buf):
    off = (-buf.data_ptr()) % 256
    return buf[off:]


class Step:
    """One layer's call configuration: problem + hyperparameters + sizes."""

    def __init__(self, q, k, v, G, S, topk, L, block_q=1, T=None, rope_theta=500000.0,
                 softmax_scale=0.0, per_q_head=False, token_segments=False):
        self.q, self.k, self.v = q, k, v
        self.prob = problem_from_tensors(q, k, v, T)
        self.par = params(G, S, topk, L, block_q, rope_theta, softmax_scale, per_q_head,
                          token_segments)
        self.sizes = query_sizes(self.prob, self.par)
        # entries per selection: topk spans, or up to topk * S tokens with token segments
        self.sel_cap = topk * S if token_segments else topk
        self.device = q.device

    @property
    def shape(self):
        """(n_q, Hq, selection heads, d): the selection heads are the KV heads,
        or the query heads when each query head selects."""
        p = self.prob
        return p.n_q, p.n_q_heads, self.sizes.n_sel_heads, p.head_dim

    def score_select(self, span_scores=False, stream=None, ws=None):
        """rea_score_select; span scores (if asked for) start as NaN, so an
        entry the library did not write shows.  ws: an aligned workspace of at
        least sizes.ws_score_select bytes to reuse, else a new one."""
        torch = _torch()
        n_q, Hq, Hkv, d = self.shape
        nb, topk = self.sizes.n_blocks, self.sel_cap
        sel = torch.empty((nb, Hkv, max(topk, 1)), dtype=torch.int32, device=self.device)
        nsel = torch.empty((nb, Hkv), dtype=torch.int32, device=self.device)
        sc = (torch.full((nb, Hkv, max(self.sizes.n_spans, 1)), float("nan"), dtype=torch.float64,
                         device=self.device) if span_scores else None)
        if ws is None:
            ws = _aligned(_ws(self.sizes.ws_score_select, self.device))
        _check(lib().rea_score_select(ctypes.byref(self.prob), ctypes.byref(self.par),
                                      _ptr(sel), _ptr(nsel), _ptr(sc), _ptr(ws),
                                      ws.numel(), _stream(stream)))
        sel = sel[:, :, :topk]
        return (sel, nsel, sc[:, :, :self.sizes.n_spans]) if span_scores else (sel, nsel)

    def gather_rope(self, sel, nsel, W_cap=None, stream=None):
        torch = _torch()
        n_q, Hq, Hkv, d = self.shape
        nb = self.sizes.n_blocks
        W_cap = int(self.sizes.W_cap if W_cap is None else W_cap)
        k_win = torch.empty((nb, Hkv, max(W_cap, 1), d), dtype=torch.float32, device=self.device)
        v_win = torch.empty((nb, Hkv, max(W_cap, 1), d), dtype=self.q.dtype, device=self.device)
        q_rot = torch.empty((n_q, Hq, d), dtype=torch.float32, device=self.device)
        W = torch.empty((nb, Hkv), dtype=torch.int32, device=self.device)
        sel_arg = sel.contiguous() if self.par.topk > 0 else None
        _check(lib().rea_gather_rope(ctypes.byref(self.prob), ctypes.byref(self.par),
                                     _ptr(sel_arg), _ptr(nsel.contiguous()), _ptr(k_win),
                                     _ptr(v_win), _ptr(q_rot), _ptr(W), W_cap, _stream(stream)))
        return k_win, v_win, q_rot, W

    def window_attend(self, q_rot, k_win, v_win, W, stream=None):
        torch = _torch()
        n_q, Hq, Hkv, d = self.shape
        out = torch.empty((n_q, Hq, d), dtype=torch.float32, device=self.device)
        W_cap = k_win.shape[2]
        # the size query covers W_cap == sizes.W_cap; scale up for larger buffers
        ratio = max(1, -(-W_cap // max(self.sizes.W_cap, 1)))
        ws = _aligned(_ws(self.sizes.ws_window_attend * ratio, self.device))
        _check(lib().rea_window_attend(ctypes.byref(self.prob), ctypes.byref(self.par), _ptr(q_rot),
                                       _ptr(k_win), _ptr(v_win), _ptr(W), W_cap, _ptr(out),
                                       _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def workspace(self):
        return _aligned(_ws(self.sizes.ws_decode_step, self.device))

    def decode_step(self, out=None, sel=None, nsel=None, ws=None, stream=None, timing=None):
        torch = _torch()
        n_q, Hq, Hkv, d = self.shape
        if out is None:
            out = torch.empty((n_q, Hq, d), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace()
        if timing is None:
            _check(lib().rea_decode_step(ctypes.byref(self.prob), ctypes.byref(self.par),
                                         _ptr(out), _ptr(sel), _ptr(nsel), _ptr(ws), ws.numel(),
                                         _stream(stream)))
        else:
            _check(lib().rea_decode_step_timed(ctypes.byref(self.prob), ctypes.byref(self.par),
                                               _ptr(out), _ptr(sel), _ptr(nsel), _ptr(ws),
                                               ws.numel(), _stream(stream),
                                               ctypes.byref(timing)))
        return out


    def decode_step_noalloc(self, out=None, sel=None, nsel=None, stream=None):
        """rea_decode_step_noalloc: the decode step on the library's fixed
        scratch array (no workspace)."""
        torch = _torch()
        n_q, Hq, Hkv, d = self.shape
        if out is None:
            out = torch.empty((n_q, Hq, d), dtype=torch.float32, device=self.device)
        _check(lib().rea_decode_step_noalloc(ctypes.byref(self.prob), ctypes.byref(self.par),
                                             _ptr(out), _ptr(sel), _ptr(nsel), _stream(stream)))
        return out


class Prefill:
    """Chunked prefill of a whole prompt: q [T][Hq][d] (every prompt token is a
    query) against the cache k, v of the same T tokens."""

    def __init__(self, q, k, v, G, S, topk, L, block_q, chunk, rope_theta=500000.0,
                 softmax_scale=0.0, per_q_head=False, token_segments=False):
        self.q, self.k, self.v = q, k, v
        self.prob = problem_from_tensors(q, k, v)
        self.par = params(G, S, topk, L, block_q, rope_theta, softmax_scale, per_q_head,
                          token_segments)
        self.chunk = chunk
        plan, self.n_blocks, self.ws_bytes = prefill_plan(self.prob, self.par, chunk,
                                                          with_blocks=True)
        self.plan = [c[:3] for c in plan]
        self.first_block = [c[3] for c in plan]
        self.n_sel_heads = self.prob.n_q_heads if per_q_head else self.prob.n_kv_heads
        self.sel_cap = topk * S if token_segments else topk
        self.device = q.device

    def workspace(self):
        return _aligned(_ws(self.ws_bytes, self.device))

    def selection_buffers(self):
        """(sel [n_blocks][H_sel][sel_cap], n_sel [n_blocks][H_sel]) int32 device
        tensors for run(); chunk c's blocks start at self.first_block[c]."""
        torch = _torch()
        sel = torch.empty((self.n_blocks, self.n_sel_heads, max(self.sel_cap, 1)),
                          dtype=torch.int32, device=self.device)
        nsel = torch.empty((self.n_blocks, self.n_sel_heads), dtype=torch.int32,
                           device=self.device)
        return sel, nsel

    def run(self, out=None, ws=None, stream=None, sel=None, nsel=None):
        torch = _torch()
        T, Hq, d = self.prob.n_q, self.prob.n_q_heads, self.prob.head_dim
        if out is None:
            out = torch.empty((T, Hq, d), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace()
        if sel is not None and (sel.shape[0] != self.n_blocks or sel.shape[2] != max(self.sel_cap, 1)
                                or not sel.is_contiguous()):
            raise ValueError("sel must be a contiguous [n_blocks][H_sel][sel_cap] tensor")
        _check(lib().rea_prefill(ctypes.byref(self.prob), ctypes.byref(self.par), self.chunk,
                                 _ptr(out), _ptr(sel), _ptr(nsel), _ptr(ws), ws.numel(),
                                 _stream(stream)))
        return out


class DecodeBatch:
    """One decode step for a batch of sequences: q [B][Hq][d], caches k, v
    [B][Hkv][T_cap][d] (or any tensors whose sequence b starts at a fixed
    stride), lengths a device int64 tensor [B] of valid tokens per sequence."""

    def __init__(self, q, k, v, lengths, G, S, topk, L, rope_theta=500000.0,
                 softmax_scale=0.0, per_q_head=False, token_segments=False):
        torch = _torch()
        if k.dim() != 4 or v.shape != k.shape or k.stride() != v.stride() or k.stride(3) != 1:
            raise ValueError("k and v must be [B][Hkv][T_cap][d] views with channel stride 1")
        if q.dim() != 3 or not q.is_contiguous() or q.shape[0] != k.shape[0]:
            raise ValueError("q must be a contiguous [B][Hq][d] tensor")
        if lengths.dtype != torch.int64 or lengths.numel() != q.shape[0] or not lengths.is_contiguous():
            raise ValueError("lengths must be a contiguous int64 tensor [B]")
        self.q, self.k, self.v, self.lengths = q, k, v, lengths
        self.batch = q.shape[0]
        # one sequence's problem: q viewed as [1][Hq][d] of sequence 0
        self.prob = problem_from_tensors(q[:1], k[0], v[0])
        self.kv_stride_seq = k.stride(0)
        self.par = params(G, S, topk, L, 1, rope_theta, softmax_scale, per_q_head, token_segments)
        self.sizes = query_sizes(self.prob, self.par)
        ws = ctypes.c_size_t()
        _check(lib().rea_decode_batch_workspace(ctypes.byref(self.prob), ctypes.byref(self.par),
                                                self.batch, ctypes.byref(ws)))
        self.ws_bytes = ws.value
        self.device = q.device

    def workspace(self):
        return _aligned(_ws(self.ws_bytes, self.device))

    def run(self, out=None, sel=None, nsel=None, ws=None, stream=None):
        torch = _torch()
        B, Hq, d = self.q.shape
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace()
        _check(lib().rea_decode_batch(ctypes.byref(self.prob), ctypes.byref(self.par), self.batch,
                                      _ptr(self.lengths), self.kv_stride_seq, _ptr(out),
                                      _ptr(sel), _ptr(nsel), _ptr(ws), ws.numel(),
                                      _stream(stream)))
        return out


def probe_stream_read(buf, wg_per_cu, loads_in_flight, sink, stream=None):
    """rea_probe_stream_read (include/rea_probe.h): stream the bytes of the
    device tensor `buf` once; sink is an int32 device tensor of at least
    wg_per_cu * CU-count elements."""
    nbytes = buf.numel() * buf.element_size()
    st = lib().rea_probe_stream_read(_ptr(buf), nbytes, wg_per_cu, loads_in_flight, _ptr(sink),
                                     _stream(stream))
    if st != 0:
        raise RuntimeError(f"rea_probe_stream_read failed ({st})")
