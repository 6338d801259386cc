"""Benchmark: ReAttention decode step on one MI355X.

Default workload: LLaMA3-8B-shaped decode at a 1,048,576-token context with all
32 layers' K/V resident in HBM (bf16, 32 q heads / 8 KV heads, d 128; G 32,
S 32, top-k 120, L 4096).  One step = rea_decode_step for each of the 32
layers (score + select + gather/RoPE + window attention), inputs resident
before the timed region.

Prints one JSON line:  value = middle-cache keys scored per second over the
whole step; ms_per_step = decode-step latency; roofline = the scoring kernel's
achieved HBM bandwidth (decode) or bf16 MFMA rate (query blocks, --config 4)
from HIP events recorded around each of its launches on the launch stream;
cpu_baseline = the CPU oracle on whole layers of the same workload.
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "middle-cache keys scored/s (achieved HBM GB/s) + decode-step latency @1M ctx"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_decode_llama8b_1m_traffic.txt")
SCORE_SRC = os.path.join(ROOT, "top_kv_cache_amd", "csrc", "score.hip")


# What the path computes in.  Decode: span scores in fp64 on the VALU (the
# scoring pass, 90% of the step), window attention in fp32; prefill blocks of
# 64: bf16 MFMA products with fp32 sums (certified, uncertain spans re-scored
# in fp64) and bf16 MFMA attention with fp32 softmax and accumulation.
DECODE_DTYPE = "f64 scoring, f32 attention"
PREFILL_DTYPE = "bf16 MFMA scoring and attention (fp32 accumulation, fp64 certification)"
DECODE_PRECISION = {"storage": "bf16", "scoring": "fp64 (VALU)", "selection": "fp64 scores",
                    "attention": "fp32 (RoPE, softmax, P.V)", "output": "fp32"}
PREFILL_PRECISION = {"storage": "bf16",
                     "scoring": "bf16 MFMA products, fp32 sums, per-span error bound",
                     "selection": "fp64 re-scoring of the spans the bound leaves uncertain",
                     "attention": "bf16 MFMA (logits from three bf16 products, P rounded to "
                                  "bf16), fp32 softmax and accumulation", "output": "fp32"}


def precision(w):
    if w.block_q == 1:
        d = dict(DECODE_PRECISION, storage=w.dtype)
        return d
    return dict(PREFILL_PRECISION, storage=w.dtype)


# selection variants of a workload (--variant)
VARIANTS = {
    "per_q_head": dict(per_q_head=True),       # one selection per query head
    "token_level": dict(S=1, topk=3840),       # spans of one token, the same token budget
    "token_segments": dict(token_segments=True),   # 120 best tokens, each widened to 32
    "pages_k127": dict(topk=127),               # the pages' 8B tuple: window exactly 8192
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (events on the launch stream)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]

    # hipEventDisableSystemFence: recording the event neither writes back nor
    # invalidates the caches at system scope, so a timed launch runs as an
    # untimed one does (a default event costs a few microseconds of idle GPU
    # on each side of the launch it brackets)
    NO_SYSTEM_FENCE = 0x20000000

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreateWithFlags(ctypes.byref(e),
                                              ctypes.c_uint(self.NO_SYSTEM_FENCE)) == 0
        return e

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def traffic_for(workload, score_bytes):
    """Measured HBM traffic per scoring launch from the committed rocprofv3 PMC
    summary, if it was taken on this workload (same name and algorithmic bytes)
    and on the current scoring kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        src = hashlib.sha256(open(SCORE_SRC, "rb").read()).hexdigest()
        if t.get("score_src_sha256") != src or t.get("workload") != workload:
            return None
        if t.get("algorithmic_bytes_per_launch") != score_bytes:
            return None
        return t["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(w, min_seconds=10.0):
    """The oracle, as it stands, on whole layers of the workload (all KV heads),
    layer after layer until at least `min_seconds` of oracle time."""
    import numpy as np
    import oracle.rea_oracle as O
    import synth
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info
                                 if p.get("user_api") == "blas"})) or blas
    except Exception:
        cores = len(os.sched_getaffinity(0))
    g = w.g
    total, layers = 0.0, 0
    for layer in range(w.n_layers):
        q64 = synth.to_f32(w.q(layer), w.dtype).astype(np.float64)
        for h in range(w.Hkv):
            K = synth.to_f32(w.kv(layer, "k", h, h + 1), w.dtype).astype(np.float64)
            V = synth.to_f32(w.kv(layer, "v", h, h + 1), w.dtype).astype(np.float64)
            t0 = time.perf_counter()
            O.step(q64[:, h * g:(h + 1) * g], K, V, w.G, w.S, w.topk, w.L, w.block_q,
                   w.rope_theta, per_q_head=w.per_q_head, token_segments=w.token_segments)
            total += time.perf_counter() - t0
            del K, V
        layers += 1
        if total >= min_seconds:
            break
    lo, hi = w.mid
    keys = (hi - lo) * w.Hkv * layers
    return {"value": keys / total, "unit": "keys/s", "cores": int(cores), "kind": "oracle",
            "blas": blas,
            "sample": f"layers 0..{layers - 1} of {w.n_layers}, all {w.Hkv} KV heads each: the "
                      f"full decode step (score, select, gather+RoPE, attend) in fp64 numpy, "
                      f"{total:.1f} s of oracle time; input generation not timed"}


def prefill_main(args):
    """Chunked prefill of one 8B-shaped layer over a prompt of args.prefill_prompt
    tokens (first G+L tokens in full, then 512-token chunks in blocks of 64):
    one JSON line with prompt tokens per second (a TTFT-style figure for one
    layer; not the headline)."""
    import torch
    import synth
    import top_kv_cache_amd as rea
    from synth import torch_io

    T = args.prefill_prompt
    w = synth.small(name=f"llama8b-bf16-prefill-prompt-{T}", seed=240715180, dtype="bf16",
                    Hq=32, Hkv=8, d=128, T=T, n_q=T, block_q=1, G=32, S=32, topk=args.topk,
                    L=4096, needles=0, kv_scaled=True)
    dev = torch.device("cuda:0")
    q = torch_io.q_device(w, 0, dev)
    K = torch_io.kv_device(w, 0, "k", device=dev)
    V = torch_io.kv_device(w, 0, "v", device=dev)
    pf = rea.Prefill(q, K, V, w.G, w.S, w.topk, w.L, 64, args.chunk, rope_theta=w.rope_theta)
    ws, out = pf.workspace(), torch.empty((T, w.Hq, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pf.run(out=out, ws=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        pf.run(out=out, ws=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] prefill of {T} tokens in {len(pf.plan)} chunks: {ms:.3f} ms "
        f"({T / ms * 1e3 / 1e6:.2f} M prompt tokens/s, one layer)")
    print(json.dumps({
        "metric": "chunked-prefill prompt tokens/s (one layer)", "value": T / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": PREFILL_DTYPE, "precision": PREFILL_PRECISION, "data": "synthetic",
        "config": {"workload": w.name, "layers": 1, "prompt": T, "chunk": args.chunk,
                   "block_q": 64, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "G": w.G, "S": w.S, "topk": w.topk, "L": w.L, "chunks": len(pf.plan)},
        "roofline": None, "cpu_baseline": None}), flush=True)


def batch_main(args):
    """Batched decode: args.batch sequences of the 8B shape, all 32 layers
    resident, one rea_decode_batch per layer; lengths all equal to
    args.context, or (--ragged) spread evenly over [context/2, context].
    One JSON line with decoded tokens per second, and the same batch run as
    one rea_decode_step per sequence and layer for comparison."""
    import torch
    import synth
    import top_kv_cache_amd as rea
    from synth import torch_io

    B, T = args.batch, args.context
    base = synth.small(name=f"llama8b-bf16-decode-batch{B}-{T // 1024}k" + ("-ragged" if args.ragged else ""),
                       seed=240715190, dtype="bf16", Hq=32, Hkv=8, d=128, T=T, n_q=1, block_q=1,
                       G=32, S=32, topk=120, L=4096, needles=4, kv_scaled=True, layers=32)
    n_layers = args.layers or 32
    dev = torch.device("cuda:0")
    lens = [T - (i * (T // 2)) // max(B - 1, 1) for i in range(B)] if args.ragged else [T] * B
    lengths = torch.tensor(lens, dtype=torch.int64, device=dev)
    t_gen = time.perf_counter()
    runs, outs, steps = [], [], []
    for layer in range(n_layers):
        q = torch.empty((B, base.Hq, base.d), dtype=torch.bfloat16, device=dev)
        K = torch.empty((B, base.Hkv, T, base.d), dtype=torch.bfloat16, device=dev)
        V = torch.empty_like(K)
        for b in range(B):
            wb = dataclasses.replace(base, seed=base.seed + 1000 * b)
            q[b] = torch_io.q_device(wb, layer, dev)[0]
            torch_io.kv_device(wb, layer, "k", out=K[b], device=dev)
            torch_io.kv_device(wb, layer, "v", out=V[b], device=dev)
        runs.append(rea.DecodeBatch(q, K, V, lengths, base.G, base.S, base.topk, base.L,
                                    rope_theta=base.rope_theta))
        steps.append([rea.Step(q[b:b + 1], K[b], V[b], base.G, base.S, base.topk, base.L, 1,
                               T=lens[b], rope_theta=base.rope_theta) for b in range(B)])
        outs.append(torch.empty((B, base.Hq, base.d), dtype=torch.float32, device=dev))
        if layer % 8 == 7 or layer == n_layers - 1:
            log(f"[bench] generated + uploaded layer {layer + 1}/{n_layers} "
                f"({time.perf_counter() - t_gen:.0f} s)")
    ws = runs[0].workspace()
    ws1 = steps[0][0].workspace()
    stream = torch.cuda.current_stream()

    def batched():
        for li in range(n_layers):
            runs[li].run(out=outs[li], ws=ws, stream=stream)

    def looped():
        for li in range(n_layers):
            for b in range(B):
                steps[li][b].decode_step(out=outs[li][b:b + 1], ws=ws1, stream=stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(batched)
    ms_loop = timed(looped)
    keys = sum(max(0, t - base.G - base.L) for t in lens) * base.Hkv * n_layers
    gbs = keys * base.d * 2 / (ms / 1e3) / 1e9
    log(f"[bench] batch of {B} at {T} tokens ({'ragged' if args.ragged else 'equal'} lengths), "
        f"{n_layers} layers: {ms:.3f} ms/step = {B / ms * 1e3:.0f} tokens/s "
        f"(middle keys at {gbs:.0f} GB/s over the whole step); one sequence at a time: "
        f"{ms_loop:.3f} ms/step ({ms_loop / ms:.2f}x slower)")
    print(json.dumps({
        "metric": "batched decode tokens/s (all layers)", "value": B / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DECODE_DTYPE, "precision": DECODE_PRECISION, "data": "synthetic",
        "config": {"workload": base.name, "layers": n_layers, "batch": B, "context": T,
                   "lengths": "ragged" if args.ragged else "equal", "q_heads": base.Hq,
                   "kv_heads": base.Hkv, "head_dim": base.d, "G": base.G, "S": base.S,
                   "topk": base.topk, "L": base.L},
        "middle_key_GBps_whole_step": gbs, "ms_per_step_one_sequence_at_a_time": ms_loop,
        "roofline": None, "cpu_baseline": None}), flush=True)


def read_ceiling_main(args):
    """HBM read ceiling: rea_probe_stream_read (the scoring kernel's load
    instruction and nothing else) over a 2 GiB buffer (or --read-mib reads
    rotating over buffers totalling 2 GiB), for 1-8 workgroups per
    CU and 4-16 loads in flight per wave; every shape timed with HIP events
    on the launch stream over args.steps launches after args.warmup.  One
    JSON line with the best rate and the table."""
    import torch
    import top_kv_cache_amd as rea

    dev = torch.device("cuda:0")
    # one read of nbytes per launch; launches rotate over a pool of at least
    # 2 GiB, so that no read finds its buffer in the 256 MB Infinity Cache
    nbytes = (args.read_mib << 20) if args.read_mib > 0 else (2 << 30)
    n_buf = max(1, -(-(2 << 30) // nbytes))
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n_buf)]
    cu = rea.lib().rea_probe_cu_count()
    sink = torch.empty(16 * cu, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    table = []
    for wpc in (1, 2, 4, 8):
        for lif in (4, 8, 16):
            for i in range(args.warmup):
                rea.probe_stream_read(bufs[i % n_buf], wpc, lif, sink, stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                rea.probe_stream_read(bufs[i % n_buf], wpc, lif, sink, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            gbs = nbytes / (us * 1e-6) / 1e9
            table.append({"wg_per_cu": wpc, "loads_in_flight": lif, "us": us, "GBps": gbs})
            log(f"[bench] read {nbytes >> 20} MiB, {wpc} workgroups/CU, {lif} loads in flight: "
                f"{us:.1f} us = {gbs:.0f} GB/s")
    best = max(table, key=lambda r: r["GBps"])
    print(json.dumps({
        "metric": "HBM streaming read ceiling (non-temporal 16-byte loads, 1 KB per wave "
                  "instruction)", "value": best["GBps"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "dtype": "u32", "data": "synthetic", "peak": HBM_PEAK_GBS,
        "frac": best["GBps"] / HBM_PEAK_GBS, "bytes": nbytes, "best": best, "table": table,
        "config": {"workload": f"stream-read-{nbytes >> 20}MiB", "buffers": n_buf, "cu": cu}}),
        flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload number (default: 1M x 32 layers)")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (exploration only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run one plain device copy of this size (HBM counter calibration)")
    ap.add_argument("--prefill-prompt", type=int, default=0,
                    help="instead: time a chunked prefill over a prompt of this many tokens")
    ap.add_argument("--chunk", type=int, default=512, help="prefill chunk (with --prefill-prompt)")
    ap.add_argument("--topk", type=int, default=120,
                    help="spans kept per block (with --prefill-prompt; the pages' setting is 127)")
    ap.add_argument("--batch", type=int, default=0,
                    help="instead: batched decode of this many sequences (8B shape, 32 layers)")
    ap.add_argument("--context", type=int, default=32768, help="sequence length (with --batch)")
    ap.add_argument("--ragged", action="store_true",
                    help="with --batch: lengths spread over [context/2, context]")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="instead: the HBM read ceiling of the scoring kernel's load pattern")
    ap.add_argument("--read-mib", type=int, default=0,
                    help="with --read-ceiling: MiB per read (default 2048; smaller reads rotate "
                         "over buffers totalling 2 GiB)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="with --config: context before the queries (T = tokens + queries)")
    ap.add_argument("--queries", type=int, default=0,
                    help="with --config: number of queries (a prefill chunk when > 1)")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default=None,
                    help="selection variant of the workload (default: one selection per KV "
                         "head over spans of S tokens)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              f"(the path is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.batch > 0:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        batch_main(args)
        return
    if args.prefill_prompt > 0 or args.read_ceiling:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        if args.read_ceiling:
            read_ceiling_main(args)
        else:
            prefill_main(args)
        return

    import torch
    import synth
    import top_kv_cache_amd as rea
    from synth import torch_io

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rea.lib()                                   # fails loudly if the library is missing
    w = synth.config(args.config)
    if args.variant:
        w = dataclasses.replace(w, **VARIANTS[args.variant])
        w.name = f"{w.name}-{args.variant.replace('_', '-')}"
    if args.tokens or args.queries:
        nq = args.queries or w.n_q
        base = args.tokens or (w.T - w.n_q)
        bq = w.block_q if nq % w.block_q == 0 else 1
        w = dataclasses.replace(w, T=base + nq, n_q=nq, block_q=bq)
        w.name = (f"{w.name.split('-')[0]}-{w.dtype}-" +
                  (f"prefill-chunk{nq}-at-{base}" if nq > 1 else f"decode-at-{base}"))
    n_layers = args.layers or w.n_layers
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: {n_layers} layers, T={w.T}, Hq={w.Hq}, Hkv={w.Hkv}, "
        f"d={w.d}, G={w.G} S={w.S} k={w.topk} L={w.L}")

    t_gen = time.perf_counter()
    steps_l, outs = [], []
    for layer in range(n_layers):
        q = torch_io.q_device(w, layer, dev)
        K = torch_io.kv_device(w, layer, "k", device=dev)
        V = torch_io.kv_device(w, layer, "v", device=dev)
        steps_l.append(rea.Step(q, K, V, w.G, w.S, w.topk, w.L, w.block_q, rope_theta=w.rope_theta,
                                per_q_head=w.per_q_head, token_segments=w.token_segments))
        outs.append(torch.empty((w.n_q, w.Hq, w.d), dtype=torch.float32, device=dev))
        if layer % 4 == 3 or layer == n_layers - 1:
            log(f"[bench] generated + uploaded layer {layer + 1}/{n_layers} "
                f"({time.perf_counter() - t_gen:.0f} s)")
    ws = steps_l[0].workspace()
    stream = torch.cuda.current_stream()
    hip = Hip()

    def one_step(timing=None):
        for li, st in enumerate(steps_l):
            st.decode_step(out=outs[li], ws=ws, stream=stream,
                           timing=timing[li] if timing is not None else None)

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n * 4} bytes done")
        del src, dst

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    # timed region: K steps, HIP events around every step and every scoring launch
    ev = [[(hip.event(), hip.event()) for _ in steps_l] for _ in range(args.steps)]
    timings = [[rea.Timing(b.value, e.value) for (b, e) in row] for row in ev]
    step_ev = [hip.event() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(step_ev[0], stream.cuda_stream)
    for s in range(args.steps):
        one_step(timings[s])
        hip.record(step_ev[s + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.elapsed_ms(step_ev[0], step_ev[-1])
    step_ms = sorted(hip.elapsed_ms(step_ev[s], step_ev[s + 1]) for s in range(args.steps))
    k1 = [hip.elapsed_ms(b, e) for row in ev for (b, e) in row]
    for row in ev:
        for (b, e) in row:
            hip.destroy(b)
            hip.destroy(e)
    for e in step_ev:
        hip.destroy(e)

    lo, hi = w.mid
    keys_per_layer = (hi - lo) * w.Hkv
    ms_per_step = total_ms / args.steps
    value = keys_per_layer * n_layers / (ms_per_step / 1e3)
    k1_ms = sum(k1) / len(k1)
    if w.block_q == 1:
        # decode: the scoring kernel streams the middle keys once
        n_scores = (hi - lo) if w.token_segments else w.n_spans
        score_bytes = (keys_per_layer * w.d * (2 if w.dtype == "bf16" else 4)
                       + n_scores * w.H_sel * 8 + w.Hq * w.d * (2 if w.dtype == "bf16" else 4))
        achieved = score_bytes / (k1_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(w.name, score_bytes),
                    "kernel": ("k_score_tokens" if (w.S == 1 or w.token_segments) else
                               "k_score_heads_mfma" if w.per_q_head else "k_score_decode"),
                    "algorithmic_bytes_per_launch": score_bytes,
                    "avg_launch_us": k1_ms * 1e3}
        log(f"[bench] scoring kernel {k1_ms * 1e3:.1f} us/launch = {achieved:.0f} GB/s "
            f"({achieved / HBM_PEAK_GBS * 100:.1f}% of {HBM_PEAK_GBS:.0f})")
    else:
        # query blocks: a bf16 GEMM of every query's group-summed vector against
        # every middle key (the kernel runs it twice, for the hi and lo halves)
        flops = 2.0 * w.n_q * keys_per_layer * w.d
        achieved = flops / (k1_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                    "kernel": "k_score_mfma", "algorithmic_flops_per_launch": flops,
                    "mfma_flops_issued_per_launch": 2 * flops, "avg_launch_us": k1_ms * 1e3}
        log(f"[bench] scoring kernel {k1_ms * 1e3:.1f} us/launch = {achieved:.0f} TFLOP/s "
            f"algorithmic, {2 * achieved:.0f} TFLOP/s issued on MFMA "
            f"({2 * achieved / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% of {MFMA_BF16_PEAK_TFLOPS:.0f})")
    med = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    p90 = step_ms[min(len(step_ms) - 1, int(0.9 * len(step_ms)))]
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}; "
        f"median {med:.3f}, p90 {p90:.3f}), {value / 1e9:.2f} G keys/s")

    res = {
        "metric": METRIC, "value": value, "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "step_ms_median": med, "step_ms_p90": p90,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DECODE_DTYPE if w.block_q == 1 else PREFILL_DTYPE,
        "precision": precision(w), "data": "synthetic",
        "config": {"workload": w.name, "layers": n_layers, "context": w.T, "batch": 1,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "storage": w.dtype,
                   "G": w.G, "S": w.S, "topk": w.topk, "L": w.L,
                   "selection": ("per query head" if w.per_q_head else "per KV head") +
                                (", token segments" if w.token_segments else ""),
                   "needles_per_kv_head": w.needles, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    del steps_l, outs, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one layer ...")
        res["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench] oracle: {res['cpu_baseline']['value'] / 1e6:.2f} M keys/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
