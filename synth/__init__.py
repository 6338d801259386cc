"""Seeded synthetic workloads for the ReAttention hot path.

Input generation only: nothing here scores, selects, rotates or attends.  The
CPU oracle (``oracle/``) and the GPU library are both fed from this module, so
they see the same inputs; the GPU receives the bytes by an upload.

Workloads stand in for the pages' long-context Needle-In-A-Haystack runs
(ReAttention, arXiv 2407.15176: the abstract's 1M/4M-token NIAH claims and the
OpenReview discussion's LLaMA3-8B-8K hyperparameter block): model-shaped heads,
Gaussian keys and values, and "needle" spans whose keys point along the
query's head-group sum, planted at random depths of the middle cache.

Random numbers: element n of a stream with key ``k`` is the n-th SplitMix64
output from state ``k`` (Steele, Lea and Flood, OOPSLA 2014).  A stream key is
itself ``sm64(seed, tensor_id << 32 | layer)``.  Gaussians come from a table of
65536 normal quantiles ``NQ[i] = fp32(Phi^-1((i + 1/2) / 65536))`` built in
fp64, indexed by the top 16 bits of the random word.

Two codings of the bulk fill exist: ``synth.c`` (OpenMP, used at scale) and
the numpy twin ``normal_block_np`` / ``needle_block_np`` (used to pin the C
code bit-for-bit on small blocks).
"""
from __future__ import annotations

import ctypes
import os
import statistics
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

# stream ids
T_Q, T_K, T_V, T_KSCALE, T_VSCALE, T_NEEDLE_POS, T_NEEDLE_NOISE = 1, 2, 3, 4, 5, 6, 7

BASE_SEED = 240715176


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# SplitMix64, scalar (python ints) and vectorised (numpy uint64, wrapping)
# ----------------------------------------------------------------------------
def sm64(key: int, n: int) -> int:
    """n-th SplitMix64 output from state `key` (python ints, mod 2**64)."""
    m = (1 << 64) - 1
    z = (key + (n + 1) * 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def sm64_np(key: int, n: np.ndarray) -> np.ndarray:
    n = n.astype(np.uint64, copy=False)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (n + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int, layer: int) -> int:
    return sm64(seed, (tensor_id << 32) | layer)


def _build_nq() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)],
                    dtype=np.float64).astype(np.float32)


NQ = _build_nq()


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (bf16 bits or fp32) -> fp32, exactly."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# numpy twin of synth.c
# ----------------------------------------------------------------------------
def normal_block_np(key, n_tok, d, h0, h1, t0, t1, scale=None, dtype="bf16"):
    h = np.arange(h0, h1, dtype=np.uint64)[:, None, None]
    t = np.arange(t0, t1, dtype=np.uint64)[None, :, None]
    c = np.arange(d, dtype=np.uint64)[None, None, :]
    with np.errstate(over="ignore"):
        ctr = (h * np.uint64(n_tok) + t) * np.uint64(d) + c
    u = sm64_np(key, ctr)
    x = NQ[(u >> np.uint64(48)).astype(np.int64)]
    if scale is not None:
        x = x * scale.reshape(-1, d)[h0:h1][:, None, :]
    x = x.astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def needle_block_np(block, key, n_tok, d, h0, h1, t0, t1, needles, length,
                    centre, noise, dtype="bf16"):
    """Overwrite needle rows of `block` ([h1-h0][t1-t0][d]) in place."""
    noise32 = np.float32(noise)
    for (hh, a0) in needles:
        if hh < h0 or hh >= h1:
            continue
        a, b = max(a0, t0), min(a0 + length, t1)
        if a >= b:
            continue
        t = np.arange(a, b, dtype=np.uint64)[:, None]
        c = np.arange(d, dtype=np.uint64)[None, :]
        ctr = (np.uint64(hh) * np.uint64(n_tok) + t) * np.uint64(d) + c
        u = sm64_np(key, ctr)
        n = (noise32 * NQ[(u >> np.uint64(48)).astype(np.int64)]).astype(np.float32)
        x = (centre.reshape(-1, d)[hh][None, :].astype(np.float32) + n).astype(np.float32)
        block[hh - h0, a - t0:b - t0] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return block


# ----------------------------------------------------------------------------
# C library
# ----------------------------------------------------------------------------
_lib = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-o", _LIB_PATH, src]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_sm64.restype = ctypes.c_uint64
        L.synth_sm64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.synth_normal.restype = None
        L.synth_normal.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.synth_needles.restype = None
        L.synth_needles.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def normal_block_c(out, key, n_tok, d, h0, h1, t0, t1, scale=None, dtype="bf16"):
    """Fill `out` ([h1-h0][t1-t0][d] view with unit channel stride) via synth.c."""
    assert out.strides[-1] == out.itemsize
    hs = out.strides[0] // out.itemsize
    rs = out.strides[1] // out.itemsize
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    lib().synth_normal(_ptr(out), 0 if dtype == "bf16" else 1, hs, rs, key, n_tok, d,
                       h0, h1, t0, t1, _ptr(NQ), None if sc is None else _ptr(sc), _threads())
    return out


def needle_block_c(out, key, n_tok, d, h0, h1, t0, t1, needles, length, centre,
                   noise, dtype="bf16"):
    if not needles:
        return out
    hs = out.strides[0] // out.itemsize
    rs = out.strides[1] // out.itemsize
    nh = np.array([n[0] for n in needles], dtype=np.int32)
    nt = np.array([n[1] for n in needles], dtype=np.int64)
    cen = np.ascontiguousarray(centre, dtype=np.float32)
    lib().synth_needles(_ptr(out), 0 if dtype == "bf16" else 1, hs, rs, key, n_tok, d,
                        h0, h1, t0, t1, _ptr(nh), _ptr(nt), length, len(needles),
                        _ptr(cen), float(noise), _ptr(NQ))
    return out


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    """One synthetic workload: shapes, hyperparameters and value recipe."""
    name: str
    seed: int
    dtype: str            # "bf16" or "f32": storage type of q, K and V
    n_layers: int
    Hq: int
    Hkv: int
    d: int
    T: int                # valid cache tokens, including the n_q newest ones
    n_q: int              # queries = the last n_q cache tokens
    block_q: int
    G: int
    S: int
    topk: int
    L: int
    needles: int = 0      # planted spans per (layer, KV head)
    kv_scaled: bool = False   # per-channel scale U(0.5, 2) on K and V
    needle_noise: float = 0.1
    rope_theta: float = 500000.0
    per_q_head: bool = False  # one selection per query head instead of per KV head
    token_segments: bool = False  # the topk best tokens, each widened to S tokens
    extra: dict = field(default_factory=dict)

    # -- derived sizes ---------------------------------------------------
    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def H_sel(self) -> int:
        """Selection heads: the KV heads, or the query heads when each selects."""
        return self.Hq if self.per_q_head else self.Hkv

    @property
    def sel_cap(self) -> int:
        """Entries of one selection: topk spans, or up to topk * S tokens."""
        return self.topk * self.S if self.token_segments else self.topk

    @property
    def g_sel(self) -> int:
        """Query heads served by one selection head."""
        return 1 if self.per_q_head else self.g

    @property
    def mid(self):
        Gp = min(self.G, self.T)
        Lp = min(self.L, self.T - Gp)
        return Gp, self.T - Lp

    @property
    def n_spans(self) -> int:
        lo, hi = self.mid
        return -(-(hi - lo) // self.S)

    @property
    def W_cap(self) -> int:
        return self.G + self.topk * self.S + self.L

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def key(self, tensor_id: int, layer: int) -> int:
        return stream_key(self.seed, tensor_id, layer)

    # -- tensors ---------------------------------------------------------
    def q(self, layer: int = 0, impl: str = "c") -> np.ndarray:
        """Queries [n_q][Hq][d] (bf16 bits or fp32), N(0,1), un-rotated."""
        key = self.key(T_Q, layer)
        n = self.n_q * self.Hq
        if impl == "np":
            x = normal_block_np(key, n, self.d, 0, 1, 0, n, None, self.dtype)
        else:
            x = np.empty((1, n, self.d), dtype=self.np_dtype)
            normal_block_c(x, key, n, self.d, 0, 1, 0, n, None, self.dtype)
        return x.reshape(self.n_q, self.Hq, self.d)

    def scale(self, which: str, layer: int):
        if not self.kv_scaled:
            return None
        tid = T_KSCALE if which == "k" else T_VSCALE
        key = self.key(tid, layer)
        u = sm64_np(key, np.arange(self.Hkv * self.d, dtype=np.uint64))
        m = (u >> np.uint64(40)).astype(np.float64)          # 24-bit integer
        return (0.5 + 1.5 * m / 16777216.0).astype(np.float32).reshape(self.Hkv, self.d)

    def needle_spans(self, layer: int):
        """[(kv_head, span index)]: distinct full spans of the middle cache."""
        if self.needles <= 0:
            return []
        lo, hi = self.mid
        n_full = (hi - lo) // self.S
        if n_full <= 0:
            return []
        key = self.key(T_NEEDLE_POS, layer)
        out = []
        for h in range(self.Hkv):
            used = set()
            for i in range(min(self.needles, n_full)):
                j = sm64(key, h * 65536 + i) % n_full
                while j in used:
                    j = (j + 1) % n_full
                used.add(j)
                out.append((h, j))
        return out

    def needle_centre(self, layer: int) -> np.ndarray:
        """fp32 [Hkv][d]: per KV head, the sequential fp32 sum of its group's
        last-query heads (the direction needle keys point along)."""
        q = to_f32(self.q(layer), self.dtype)[-1]           # [Hq][d]
        c = np.zeros((self.Hkv, self.d), dtype=np.float32)
        for h in range(self.Hkv):
            acc = q[h * self.g].astype(np.float32)
            for gg in range(1, self.g):
                acc = (acc + q[h * self.g + gg]).astype(np.float32)
            c[h] = acc
        return c

    def _needle_rows(self, layer):
        lo, _ = self.mid
        return [(h, lo + j * self.S) for (h, j) in self.needle_spans(layer)]

    def kv(self, layer: int, which: str, h0: int = 0, h1: int | None = None,
           t0: int = 0, t1: int | None = None, out: np.ndarray | None = None,
           impl: str = "c") -> np.ndarray:
        """Cache block [h1-h0][t1-t0][d] of K (which='k') or V ('v')."""
        h1 = self.Hkv if h1 is None else h1
        t1 = self.T if t1 is None else t1
        tid = T_K if which == "k" else T_V
        key = self.key(tid, layer)
        sc = self.scale(which, layer)
        if impl == "np":
            blk = normal_block_np(key, self.T, self.d, h0, h1, t0, t1, sc, self.dtype)
            if which == "k" and self.needles:
                needle_block_np(blk, self.key(T_NEEDLE_NOISE, layer), self.T, self.d,
                                h0, h1, t0, t1, self._needle_rows(layer), self.S,
                                self.needle_centre(layer), self.needle_noise, self.dtype)
            if out is not None:
                out[...] = blk
                return out
            return blk
        if out is None:
            out = np.empty((h1 - h0, t1 - t0, self.d), dtype=self.np_dtype)
        normal_block_c(out, key, self.T, self.d, h0, h1, t0, t1, sc, self.dtype)
        if which == "k" and self.needles:
            needle_block_c(out, self.key(T_NEEDLE_NOISE, layer), self.T, self.d,
                           h0, h1, t0, t1, self._needle_rows(layer), self.S,
                           self.needle_centre(layer), self.needle_noise, self.dtype)
        return out


def config(i: int) -> Workload:
    """The five evaluation workloads (sizes as the configuration list states)."""
    s = BASE_SEED + i
    if i == 1:
        return Workload("tiny-f32-decode-4k", s, "f32", 1, 2, 1, 64, 4096, 1, 1,
                        4, 16, 8, 64, needles=1)
    if i == 2:
        return Workload("llama8b-bf16-decode-128k", s, "bf16", 1, 32, 8, 128, 131072, 1, 1,
                        32, 32, 120, 4096, needles=4, kv_scaled=True)
    if i == 3:
        return Workload("llama8b-bf16-decode-1m-32layers", s, "bf16", 32, 32, 8, 128,
                        1048576, 1, 1, 32, 32, 120, 4096, needles=8, kv_scaled=True)
    if i == 4:
        return Workload("llama8b-bf16-prefill-chunk4096-at-128k", s, "bf16", 1, 32, 8, 128,
                        131072 + 4096, 4096, 64, 32, 32, 120, 4096)
    if i == 5:
        return Workload("llama3b-bf16-decode-4m", s, "bf16", 1, 24, 8, 128, 4194304, 1, 1,
                        32, 64, 256, 16000, needles=16)
    raise ValueError(i)


def small(name="small", seed=7, dtype="bf16", Hq=4, Hkv=2, d=64, T=700, n_q=1, block_q=1,
          G=4, S=16, topk=5, L=64, needles=1, kv_scaled=False, layers=1,
          per_q_head=False, token_segments=False) -> Workload:
    """A shrunken workload with the same recipe, for quick tests."""
    return Workload(name, seed, dtype, layers, Hq, Hkv, d, T, n_q, block_q, G, S, topk, L,
                    needles=needles, kv_scaled=kv_scaled, per_q_head=per_q_head,
                    token_segments=token_segments)
