"""Upload generated workloads into device tensors (input plumbing only).

Host generation (synth.c) writes into a pinned staging buffer a head at a
time; the buffer is then copied into the device tensor.  The bytes on the
device are exactly the bytes the CPU oracle is given.
"""
import numpy as np
import torch

from . import Workload, to_f32


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _staging_view(t: torch.Tensor, w: Workload) -> np.ndarray:
    if w.dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def q_device(w: Workload, layer: int = 0, device="cuda") -> torch.Tensor:
    q = w.q(layer)
    t = torch.from_numpy(q.view(np.int16) if w.dtype == "bf16" else q)
    if w.dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device).contiguous()


def kv_device(w: Workload, layer: int, which: str, out: torch.Tensor = None,
              device="cuda", rows_per_chunk: int = 1 << 21) -> torch.Tensor:
    """Fill (or allocate) a [Hkv][T][d] device tensor with K ('k') or V ('v')."""
    if out is None:
        out = torch.empty((w.Hkv, w.T, w.d), dtype=torch_dtype(w), device=device)
    chunk = min(rows_per_chunk, w.T)
    stage = torch.empty((1, chunk, w.d), dtype=torch_dtype(w), pin_memory=True)
    sv = _staging_view(stage, w)
    for h in range(w.Hkv):
        for t0 in range(0, w.T, chunk):
            t1 = min(t0 + chunk, w.T)
            w.kv(layer, which, h, h + 1, t0, t1, out=sv[:, :t1 - t0])
            out[h:h + 1, t0:t1].copy_(stage[:, :t1 - t0], non_blocking=False)
    return out


def as_f64(x: np.ndarray, w: Workload) -> np.ndarray:
    return to_f32(x, w.dtype).astype(np.float64)
