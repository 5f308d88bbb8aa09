"""Throughput of the LLaMA hot path on one MI355X.

One step = one pass of the whole path over synthetic seeded inputs:
  * prefill: one LLaMA-7B-shape block (d 4096, 32 heads, hidden 11008) over
    one sequence of 2048 tokens, bf16 weights/activations, fp32 accumulate;
  * decode: one step of the whole LLaMA-7B-shape model (32 blocks, final norm,
    32000-wide head) for 32 sequences at position 2047 over a seeded KV cache,
    replayed as a HIP graph.
`value` is prefill tokens/s; decode tokens/s and both roofline fractions are
reported beside it. Inputs are resident in HBM before timing starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector peak
COPY_CALIBRATION_BYTES = 1 << 30   # bytes read and written by each calibration copy

# HBM bytes per launch of the roofline kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (decoder_only_transformer_llama_amd/profile_summary.py);
# reported only while the kernel sources match the ones profiled.
TRAFFIC_PROFILES = {
    "gate_up": os.path.join(ROOT, "profiles", "gemm_gate_up_7b_s2048_traffic.txt"),
    "dec_attn": os.path.join(ROOT, "profiles", "dec_attn_7b_decode_b32_traffic.txt"),
}


def stored_traffic(key: str):
    from decoder_only_transformer_llama_amd.profile_summary import stored_traffic as st
    v = st(TRAFFIC_PROFILES[key])
    return None if v is None else round(v)


def decode_summary(dec: dict) -> dict:
    return {
        "workload": "llama-7b-shape model decode step, batch 32, KV cache 2047 positions, bf16",
        "tokens_per_s": round(dec["tokens_per_s"], 1), "ms_per_step": round(dec["ms"], 4),
        "ms_per_step_eager": round(dec["ms_eager"], 4), "hip_graph": dec["graph"],
        "hbm_gbs": round(dec["hbm_gbs"], 1), "hbm_frac": round(dec["hbm_gbs"] / PEAK_HBM_GBS, 4),
        "bytes_per_step": dec["bytes"], "roofline": dec["roofline"], "kernels_ms": dec["per_kernel_ms"],
    }


def copy_calibration(torch) -> None:
    """A plain device copy of known size (read and write COPY_CALIBRATION_BYTES
    each) for scaling the HBM byte counters; run under rocprofv3 --pmc."""
    n = COPY_CALIBRATION_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(f"# copy calibration: 3 copies of {COPY_CALIBRATION_BYTES} bytes (kernel MulFunctor)", flush=True)


class HipEvents:
    """hipEvent_t handles via the HIP runtime (timing on the library's stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            rc = self.hip.hipEventCreate(ctypes.byref(self.ev, i * ctypes.sizeof(ctypes.c_void_p)))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
        self.n = n

    def record(self, i: int, stream) -> None:
        self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream))

    def elapsed_ms(self, a: int, b: int) -> float:
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b]))
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def pointer_from(self, i: int):
        return ctypes.cast(ctypes.byref(self.ev, i * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))


def block_flops(w) -> dict:
    n, d, h, S, B = w.tokens, w.dim, w.hidden, w.seq, w.batch
    return {
        "qkv": 2.0 * n * d * 3 * d,
        "attention": 2.0 * d * S * (S + 1) * B,       # unmasked (q, k) pairs incl. the diagonal, QK^T + PV
        "o": 2.0 * n * d * d,
        "gate_up": 2.0 * n * d * 2 * h,
        "down": 2.0 * n * h * d,
    }


def decode_bytes(w) -> dict:
    d, h, L, B, V, P, kvd = w.dim, w.hidden, w.n_layers, w.batch, w.vocab, w.decode_pos, w.kv_dim
    return {
        "weights": L * ((2 * d + 2 * kvd) * d + 3 * d * h) * 2 + V * d * 2,
        "kv_read": L * B * P * kvd * 2 * 2,
        "kv_write": L * B * kvd * 2 * 2,
        "embed_logits": B * d * 2 + B * V * 4,
    }


def traced_kernel_ms(lib, run, stream, reps: int, capacity: int = 4096):
    """Per-kernel durations (ms) averaged over `reps` traced runs of `run`, as
    a list of (library step label, ms). An untraced run goes first so the GPU
    is busy while the traced run is enqueued: the first traced kernel then
    starts as soon as the start event completes, and its time holds no host
    launch latency."""
    ev = HipEvents(capacity + 1)
    tot, labels = None, None
    for _ in range(reps):
        run()
        ev.record(0, stream)
        lib.llama_trace_begin(ev.pointer_from(1), capacity)
        run()
        got = lib.llama_trace_end()
        if got >= capacity:
            raise RuntimeError("trace capacity exhausted")
        lab = [lib.llama_trace_label(i).decode() for i in range(got)]
        if labels is None:
            labels, tot = lab, [0.0] * got
        elif lab != labels:
            raise RuntimeError("launch sequence changed between traced runs")
        for i in range(got):
            tot[i] += ev.elapsed_ms(i, i + 1)
    return [(l, t / reps) for l, t in zip(labels, tot)]


def merge_steps(trace, names):
    """Sum consecutive kernels of one library step; map labels to short names."""
    out = []
    for label, ms in trace:
        n = names.get(label, label)
        if out and out[-1][0] == n:
            out[-1] = (n, out[-1][1] + ms)
        else:
            out.append((n, ms))
    return out


PREFILL_STEP_NAMES = {
    "attention norm": "attn_norm", "rope table": "rope_table", "qkv projection": "qkv", "attention": "attention",
    "output projection": "o", "ffn norm": "ffn_norm", "gate/up projection": "gate_up", "down projection": "down",
    "down residual": "down_reduce",
}


def bench_prefill(args, torch):
    from decoder_only_transformer_llama_amd import _lib, inputs as I
    from decoder_only_transformer_llama_amd.workloads import block_workload

    bw = block_workload(1, "cuda", numerics=args.numerics, weights_f16=not args.bf16_weights)
    w = bw.w
    stream = torch.cuda.current_stream().cuda_stream
    run = lambda: bw.block(bw.x)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(args.steps):
        run()
    ev.record(1, stream)
    ms_eager = ev.elapsed_ms(0, 1) / args.steps
    torch.cuda.synchronize()
    # the block's launches captured once into a HIP graph and replayed, timed
    # beside the eager launches (which are the reported figure: on this stack
    # the graph replay of these ten kernels measured ~2% slower)
    graph = None
    if not args.eager:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                run()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                run()
            torch.cuda.synchronize()
        except Exception as e:  # pragma: no cover - reported, eager timing still valid
            print(f"# prefill graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph = None
    ms, ms_graph = ms_eager, None
    if graph is not None:
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ev.record(0, stream)
        for _ in range(args.steps):
            graph.replay()
        ev.record(1, stream)
        ms_graph = ev.elapsed_ms(0, 1) / args.steps
        torch.cuda.synchronize()

    trace = traced_kernel_ms(_lib.load(), lambda: bw.block(bw.x), stream, max(3, args.steps // 2))
    if args.raw_trace:
        print("# prefill kernels: " + json.dumps([(l, round(t, 4)) for l, t in trace]), file=sys.stderr, flush=True)
    steps = merge_steps(trace, PREFILL_STEP_NAMES)
    names, kms = [n for n, _ in steps], [t for _, t in steps]
    fl = block_flops(w)
    total = sum(fl.values())
    per_kernel = {n: {"ms": round(t, 4)} for n, t in zip(names, kms)}
    for n in fl:
        per_kernel[n]["tflops"] = round(fl[n] / (kms[names.index(n)] * 1e-3) / 1e12, 1)
        per_kernel[n]["mfma_frac"] = round(per_kernel[n]["tflops"] / PEAK_BF16_TFLOPS, 4)
    dom = "gate_up"
    achieved = fl[dom] / (kms[names.index(dom)] * 1e-3) / 1e12
    return {
        "w": w, "ms": ms, "ms_graph": ms_graph, "tokens_per_s": w.tokens / (ms * 1e-3),
        "block_tflops": total / (ms * 1e-3) / 1e12,
        "per_kernel": per_kernel,
        # the gate/up GEMM runs as its launches of one step: whole rounds of
        # 256 x 256 tiles, then (7B) the last round's columns as 192 x 256 tiles
        "roofline": {"bound": "mfma", "kernel": "gate/up GEMM (fp16 h*g2 x fp16 weights on the fp16 matrix cores; "
                                                "rstd row scale + SiLU*up epilogue; 256- and 192-row tile launches)"
                     if not args.bf16_weights else
                     "gate/up GEMM (fp16 h*g2 x bf16 weights converted in registers; rstd row scale + SiLU*up "
                     "epilogue; 256- and 192-row tile launches)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": stored_traffic("gate_up"),
                     "flops_per_launch": fl[dom]},
        "block": bw,
    }


def bench_other_blocks(args, torch):
    """Throughput of the 13B-shape (4 x 2048 tokens) and 65B-shape (2 x 2048)
    block prefill workloads, reported beside the headline (fraction of the
    bf16 matrix-core peak)."""
    from decoder_only_transformer_llama_amd.workloads import block_workload
    out = {}
    for wid in (2, 3):
        bw = block_workload(wid, "cuda", weights_f16=not args.bf16_weights)
        w = bw.w
        for _ in range(max(1, args.warmup // 2)):
            bw.block(bw.x)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        reps = max(2, args.steps // 2)
        ev = HipEvents(2)
        ev.record(0, stream)
        for _ in range(reps):
            bw.block(bw.x)
        ev.record(1, stream)
        ms = ev.elapsed_ms(0, 1) / reps
        torch.cuda.synchronize()
        tf = sum(block_flops(w).values()) / (ms * 1e-3) / 1e12
        out[w.name] = {"ms": round(ms, 3), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1), "tflops": round(tf, 1),
                       "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del bw
        torch.cuda.empty_cache()
    return out


def time_block(torch, bw, reps: int, warmup: int) -> float:
    """Mean ms of bw.block(bw.x) over `reps` calls (HIP events on the library's stream)."""
    for _ in range(warmup):
        bw.block(bw.x)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(reps):
        bw.block(bw.x)
    ev.record(1, stream)
    ms = ev.elapsed_ms(0, 1) / reps
    torch.cuda.synchronize()
    return ms


def bench_extra_blocks(args, torch):
    """The 7B-shape block with bf16 matrix-core projections (bf16 operands and
    weights, no fp16 copies) beside the default, and the tiny fp32 block
    (d 256, 128 tokens: launch-bound, no roofline target)."""
    from decoder_only_transformer_llama_amd import _lib as L
    from decoder_only_transformer_llama_amd.workloads import block_workload
    # every projection operand one bf16 value on the bf16 matrix cores, the
    # attention output into Wo as a bf16 hi/lo pair, fp16 attention
    bf16_operands = L.NUM_EXPLICIT | L.NUM_ATTN_F16 | L.NUM_O_A_PAIR
    out = {}
    bw = block_workload(1, "cuda", numerics=bf16_operands)
    ms = time_block(torch, bw, args.steps, args.warmup)
    tf = sum(block_flops(bw.w).values()) / (ms * 1e-3) / 1e12
    out["7b-block-bf16-operands"] = {"ms": round(ms, 4), "tokens_per_s": round(bw.w.tokens / (ms * 1e-3), 1),
                                     "tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                     "numerics": hex(bf16_operands)}
    del bw
    torch.cuda.empty_cache()
    bw = block_workload(0, "cuda")
    ms = time_block(torch, bw, args.steps, args.warmup)
    out[bw.w.name] = {"ms": round(ms, 4), "tokens_per_s": round(bw.w.tokens / (ms * 1e-3), 1),
                      "tflops": round(sum(block_flops(bw.w).values()) / (ms * 1e-3) / 1e12, 3)}
    return out


def bench_train_step(args, torch, wid: int = 0):
    """fp32 training step of a block (forward keeping the linear outputs,
    manual backward, SGD update of all nine weights) on an fp32 block workload
    (the tiny block, or the d1024 seq-1024 block). Work is counted as three
    times the forward's matrix products (the backward's input and weight
    gradients are two more of each)."""
    from decoder_only_transformer_llama_amd import inputs as I, ops
    w = I.workload(wid)
    wt = I.block_weights(w, device="cuda")
    x = I.block_input(w, device="cuda")
    t = I.normal((w.tokens, w.dim), w.wid, 0, I.T_BUMP, device="cuda")
    cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=torch.float32, eps=w.eps, theta=w.theta)
    tb = ops.TrainBlock(cfg, wt, w.batch, w.seq)
    for _ in range(args.warmup):
        tb.train_step(x, t, 1e-6)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(args.steps):
        tb.train_step(x, t, 1e-6)
    ev.record(1, stream)
    ms = ev.elapsed_ms(0, 1) / args.steps
    torch.cuda.synchronize()
    fl = 3 * sum(block_flops(w).values())
    return {"workload": f"{w.name}: fp32 block training step (forward, backward, SGD), batch {w.batch}, seq {w.seq}",
            "ms": round(ms, 4), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2), "fp32_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}


def bench_decode(args, torch, wid: int = 4, with_model_prefill: bool = True):
    from decoder_only_transformer_llama_amd import _lib
    from decoder_only_transformer_llama_amd.workloads import decode_workload

    wl = decode_workload(wid, "cuda")
    w = wl.w
    m = wl.model
    logits = torch.empty((w.batch, w.vocab), dtype=torch.float32, device="cuda")
    run = lambda: m.decode(wl.tokens, wl.pos, wl.k_cache, wl.v_cache, logits)
    run()
    torch.cuda.synchronize()
    graph = None
    try:
        if args.eager:
            raise RuntimeError("--eager")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
    except Exception as e:  # pragma: no cover - reported, eager timing still valid
        if not args.eager:
            print(f"# decode graph capture failed ({e}); timing eager launches", file=sys.stderr)
        graph = None
    step = graph.replay if graph is not None else run
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(args.steps):
        step()
    ev.record(1, stream)
    ms = ev.elapsed_ms(0, 1) / args.steps
    # eager timing too (launch overhead visible)
    ev.record(0, stream)
    for _ in range(max(2, args.steps // 4)):
        run()
    ev.record(1, stream)
    ms_eager = ev.elapsed_ms(0, 1) / max(2, args.steps // 4)

    L = w.n_layers
    names = {"rope table": "rope_table", "embedding": "embed", "qkv projection": "qkv", "attention": "attention",
             "output projection": "o", "attention residual": "resid1", "gate/up projection": "gate_up",
             "silu": "silu", "down projection": "down", "ffn residual": "resid2", "output head": "head",
             "head combine": "head_combine"}
    agg = {}
    for label, t in traced_kernel_ms(_lib.load(), run, stream, 2):
        n = names.get(label, label)
        agg[n] = agg.get(n, 0.0) + t
    by = decode_bytes(w)
    total_bytes = sum(by.values())
    att_bytes_launch = by["kv_read"] / L
    att_ms = agg["attention"] / L
    achieved = att_bytes_launch / (att_ms * 1e-3) / 1e9
    model_prefill = None if (args.no_model_prefill or not with_model_prefill) else bench_model_prefill(args, torch, wl)
    return {
        "w": w, "ms": ms, "ms_eager": ms_eager, "graph": graph is not None, "model_prefill": model_prefill,
        "tokens_per_s": w.batch / (ms * 1e-3),
        "hbm_gbs": total_bytes / (ms * 1e-3) / 1e9,
        "bytes": total_bytes,
        "per_kernel_ms": {k: round(v, 4) for k, v in agg.items()},
        "roofline": {"bound": "hbm", "kernel": "dec_attn (fused q/k/v finish, RoPE, cache append, attention)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": stored_traffic("dec_attn"),
                     "bytes_per_launch": att_bytes_launch},
    }


def bench_model_prefill(args, torch, wl, seq: int = 2048):
    """Whole-model prefill on the decode workload's 7B-shape model: one
    sequence of `seq` seeded tokens through 32 blocks (filling a KV cache),
    the final norm and the 32000-wide head."""
    from decoder_only_transformer_llama_amd import inputs as I
    from decoder_only_transformer_llama_amd import ops
    w, m = wl.w, wl.model
    if not args.bf16_weights:
        # the same model with its projections and head as fp16 (converted once;
        # the decode pack and the bf16 weights stay for the decode legs)
        num, layers = args.numerics, []
        for lw in m.layers:
            num_l, l16 = ops.with_f16_weights(args.numerics, lw)
            layers.append(l16)
            num = num_l
        cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=w.torch_dtype, n_layers=w.n_layers, vocab=w.vocab,
                         max_seq=w.max_seq, eps=w.eps, theta=w.theta, numerics=num, n_kv_heads=w.n_kv_heads)
        tok_emb, final_norm, head = m.tensors
        m = ops.Model(cfg, layers, tok_emb, final_norm, ops.convert_weights_f16(head))
    toks = I.tokens(w, (1, seq), device="cuda", stream=1)
    kc, vc = m.new_cache(1, "cuda"), m.new_cache(1, "cuda")
    for _ in range(max(1, args.warmup // 2)):
        m.forward(toks, kc, vc)
    torch.cuda.synchronize()
    reps = max(2, args.steps // 4)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(reps):
        m.forward(toks, kc, vc)
    ev.record(1, stream)
    ms = ev.elapsed_ms(0, 1) / reps
    torch.cuda.synchronize()
    blk = block_flops(type("W", (), {"tokens": seq, "dim": w.dim, "hidden": w.hidden, "seq": seq, "batch": 1}))
    flops = w.n_layers * sum(blk.values()) + 2.0 * seq * w.dim * w.vocab
    del kc, vc, m
    return {"workload": f"llama-7b-shape model prefill, 32 blocks + head, batch 1, seq {seq}, bf16",
            "ms": round(ms, 3), "tokens_per_s": round(seq / (ms * 1e-3), 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(bw, torch, budget_s: float = 10.0, max_reps: int = 8):
    """The fp64 oracle on the host: the whole 2048-token 7B-shape block
    forward, repeated until about `budget_s` seconds of CPU work (at most
    `max_reps` passes), reported as tokens/s over all passes."""
    import numpy as np
    from oracle import llama_oracle as O
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in info if p.get("user_api") == "blas") \
            or blas
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    w = bw.w
    x = O.f64(bw.x.cpu())
    wt = {k: O.f64(v.cpu()) for k, v in bw.weights.items()}
    reps, t0 = 0, time.perf_counter()
    while True:
        O.block_forward(x, wt, w.batch, w.seq, w.n_heads, w.eps, w.theta)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= max_reps:
            break
    return {"value": round(reps * w.tokens / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"7B-shape block forward (fp64 NumPy oracle), batch {w.batch} x seq {w.seq}, "
                      f"{reps} pass(es) in {dt:.2f} s",
            "cpu_model": cpu_model, "blas": blas}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="skip the prefill leg (diagnostic runs)")
    ap.add_argument("--eager", action="store_true", help="decode: time eager launches, no HIP graph")
    ap.add_argument("--raw-trace", action="store_true", help="print every traced prefill kernel's time")
    ap.add_argument("--no-model-prefill", action="store_true", help="skip the whole-model prefill leg")
    ap.add_argument("--no-other-blocks", action="store_true", help="skip the 13B/65B-shape block legs")
    ap.add_argument("--no-gqa-decode", action="store_true", help="skip the grouped-query decode leg")
    ap.add_argument("--no-train", action="store_true", help="skip the fp32 training-step leg")
    ap.add_argument("--train-only", action="store_true", help="only the fp32 training-step legs (diagnostic runs)")
    ap.add_argument("--bf16-weights", action="store_true",
                    help="prefill: keep the projections' weights bf16 and convert them in registers at every "
                         "product, instead of fp16 copies made once (same output bits)")
    ap.add_argument("--numerics", type=lambda v: int(v, 0), default=0,
                    help="prefill operand-precision bits (llama_config.numerics; 0 = library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain copy used to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the hot path here runs on a single MI355X with no sharding or "
              "collectives; --gpus above 1 is not supported.", file=sys.stderr)
        return 2
    import torch
    torch.cuda.set_device(0)
    t_start = time.time()
    if args.copy_calibration:
        copy_calibration(torch)
        return 0
    if args.train_only:
        for wid in (0, 8):
            print(f"# train step: {json.dumps(bench_train_step(args, torch, wid))}", file=sys.stderr, flush=True)
        return 0
    if args.decode_only:
        dec = bench_decode(args, torch)
        print(f"# decode: {dec['ms']:.3f} ms/step (eager {dec['ms_eager']:.3f}), {dec['tokens_per_s']:.0f} tok/s, "
              f"{dec['hbm_gbs']:.0f} GB/s; kernels {json.dumps(dec['per_kernel_ms'])}", file=sys.stderr, flush=True)
        # the decode object of the full line on its own (diagnostic runs: profiles read its roofline)
        print(json.dumps({"decode": decode_summary(dec)}), flush=True)
        if dec["model_prefill"]:
            print(f"# model prefill: {json.dumps(dec['model_prefill'])}", file=sys.stderr, flush=True)
        if not args.no_gqa_decode:
            torch.cuda.empty_cache()
            g = bench_decode(args, torch, wid=5, with_model_prefill=False)
            print(f"# gqa decode: {g['ms']:.3f} ms/step, {g['tokens_per_s']:.0f} tok/s, {g['hbm_gbs']:.0f} GB/s; "
                  f"kernels {json.dumps(g['per_kernel_ms'])}", file=sys.stderr, flush=True)
        return 0
    pf = bench_prefill(args, torch)
    print(f"# prefill: {pf['ms']:.3f} ms/step, {pf['tokens_per_s']:.0f} tok/s, block {pf['block_tflops']:.1f} "
          f"TFLOP/s; kernels {json.dumps(pf['per_kernel'])}", file=sys.stderr, flush=True)
    others = None
    if not args.prefill_only and not args.no_other_blocks:
        others = bench_other_blocks(args, torch)
        print(f"# other blocks: {json.dumps(others)}", file=sys.stderr, flush=True)
        others.update(bench_extra_blocks(args, torch))
        print(f"# extra blocks: {json.dumps(others)}", file=sys.stderr, flush=True)
    dec = None
    if not args.prefill_only:
        dec = bench_decode(args, torch)
        print(f"# decode: {dec['ms']:.3f} ms/step (eager {dec['ms_eager']:.3f}), {dec['tokens_per_s']:.0f} tok/s, "
              f"{dec['hbm_gbs']:.0f} GB/s; kernels {json.dumps(dec['per_kernel_ms'])}", file=sys.stderr, flush=True)
        if dec["model_prefill"]:
            print(f"# model prefill: {json.dumps(dec['model_prefill'])}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    gqa = None
    if not args.prefill_only and not args.no_gqa_decode:
        g = bench_decode(args, torch, wid=5, with_model_prefill=False)
        gqa = {"workload": "llama-7b-shape model decode step with 8 key/value heads (groups of 4), batch 32, "
                           "KV cache 2047 positions, bf16",
               "tokens_per_s": round(g["tokens_per_s"], 1), "ms_per_step": round(g["ms"], 4),
               "hbm_gbs": round(g["hbm_gbs"], 1), "hbm_frac": round(g["hbm_gbs"] / PEAK_HBM_GBS, 4),
               "bytes_per_step": g["bytes"], "attention_gbs": g["roofline"]["achieved"],
               "kernels_ms": g["per_kernel_ms"]}
        print(f"# gqa decode: {json.dumps(gqa)}", file=sys.stderr, flush=True)
    train = None
    if not args.prefill_only and not args.no_train:
        train = [bench_train_step(args, torch, wid) for wid in (0, 8)]
        for tr in train:
            print(f"# train step: {json.dumps(tr)}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(pf["block"], torch)
    w = pf["w"]
    line = {
        "metric": "prefill tokens/s (7B block, seq 2048) + decode tokens/s; % of roofline",
        "value": round(pf["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms"], 4),
        "ms_per_step_hip_graph": None if pf["ms_graph"] is None else round(pf["ms_graph"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp16",
        "data": "synthetic",
        "config": {"workload": "llama-7b-shape block prefill, batch 1, seq 2048, bf16 (fp32 accumulate)",
                   "dim": w.dim, "n_heads": w.n_heads, "hidden": w.hidden, "batch": w.batch, "seq": w.seq,
                   "weights": ("bf16, converted to fp16 in registers at each product" if args.bf16_weights else
                               "bf16 model; projections stored as fp16 copies made once before timing "
                               "(output bit-identical to converting in registers)"),
                   "parallelism": "single GPU"},
        "block_mfma_frac": round(pf["block_tflops"] / PEAK_BF16_TFLOPS, 4),
        "block_tflops": round(pf["block_tflops"], 1),
        "roofline": pf["roofline"],
        "prefill_kernels": pf["per_kernel"],
        "other_blocks": others,
        "cpu_baseline": cpu,
    }
    if dec is not None:
        dw = dec["w"]
        line["decode"] = decode_summary(dec)
        if dec["model_prefill"] is not None:
            line["model_prefill"] = dec["model_prefill"]
    if gqa is not None:
        line["decode_gqa"] = gqa
    if train is not None:
        line["train_step"] = train
    line["wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
