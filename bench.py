#!/usr/bin/env python3
"""Throughput of the gated delta-rule mixer on one MI355X.

Headline (the JSON line's ``value``): decode state-stream bandwidth of the GDN
decode step, B=64 sequences x H=32 heads x dk=dv=128, over 48 independent
layer states (6 GiB of fp32 state, far beyond the on-chip caches).  One
"step" is one decoded token for every sequence: 48 back-to-back
``gdr_decode_step`` calls on one stream, each streaming its 128 MiB state
in and out.  ``value`` = algorithmic bytes moved per step x steps / elapsed.

Also measured in the same run (under ``workloads``): KDA decode (B=256,
20 in-place steps), GDN chunked prefill (B=4, T=8192) and KDA chunked
prefill (B=1, T=32768), each with its roofline fractions.

The headline step is captured once as a HIP graph (48 kernel launches) and
replayed, so the timed region holds GPU work only.  Roofline: algorithmic
bytes (or flops) per launch divided by the average launch duration, from HIP
events recorded around the timed region on the stream the kernels run on
(GPU time / launches in the region).  ``cpu_baseline`` times the float64 CPU oracle on a
bounded sample of the headline workload; the KDA decode, the small fp32 case
and both prefills carry their own ``cpu_baseline``: the oracle's full run on
the same inputs, with the host's core count and CPU model.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
       [--no-cpu-baseline] [--launches N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode state-stream GB/s vs HBM peak; chunked-prefill tokens/s vs MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector peak
CHUNK = 64


def decode_bytes_per_head(gate, dk, dv, elt=2):
    """Read + write the fp32 state, read q, k, v, write o, read the gates."""
    return 8 * dk * dv + elt * (2 * dk + 2 * dv) + 4 + (4 * dk if gate == "kda" else 4)


def verify_bytes_per_head(gate, dk, dv, T, save, elt=2):
    """Multi-token decode of T tokens: read + write the fp32 state once, write
    the T intermediate states if kept, and each token's q, k, v, o and gates."""
    per_tok = elt * (2 * dk + 2 * dv) + 4 + (4 * dk if gate == "kda" else 4)
    return 8 * dk * dv + (4 * dk * dv * T if save else 0) + T * per_tok


def decode_flops_per_head(dk, dv):
    return 7 * dk * dv


def prefill_bytes(gate, B, T, H, dk, dv, has_s0, elt=2):
    per_tok = elt * (2 * dk + 2 * dv) + 4 + (4 * dk if gate == "kda" else 4)
    return B * T * H * per_tok + B * H * 4 * dk * dv * (2 if has_s0 else 1)


def prefill_flops(B, T, H, dk, dv):
    """Matrix-core flops of the chunked algorithm per token-head (C = 64): the
    intra-chunk products (A, P, W, U-tilde) 2C(3dk + 2dv) plus the inter-chunk
    state products (W S, Qhat S, Ktil^T U) 6 dk dv."""
    return B * T * H * (2 * CHUNK * (3 * dk + 2 * dv) + 6 * dk * dv)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_08_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, sha):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on this exact kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        e = d.get(kernel_key)
        if e and e.get("source_sha256") == sha:
            return e.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the oracle figures."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def oracle_baseline(run, units, unit, sample, gpu_rate, reps=1):
    """Times ``run(nthreads)`` (the float64 oracle on the workload's own
    inputs, ``reps`` times) on every host core visible to the process; the
    rate is ``units`` per run per second.  A baseline, not a target."""
    import oracle
    nt = oracle.default_threads()
    t0 = time.perf_counter()
    for _ in range(reps):
        run(nt)
    dt = (time.perf_counter() - t0) / reps
    v = units / dt
    return {"value": round(v, 3), "unit": unit, "cores": nt, "kind": "oracle", "sample": sample,
            "seconds": round(dt, 6), "cpu": cpu_model(),
            "gpu_over_oracle": round(gpu_rate / v, 1) if gpu_rate else None}


def c_decode_call(torch, gdr, gate, d, scale=1.0):
    """A zero-argument callable that enqueues one gdr_decode_step through the C
    ABI with pre-marshalled pointers on the current stream (no per-call Python
    checks, so the host stays ahead of the GPU)."""
    import ctypes
    lib = gdr.load_library()
    B, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dtype = 1 if d["q"].dtype == torch.bfloat16 else 0
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    args = (gdr.GATES[gate], dtype, B, H, dk, dv, ctypes.c_float(scale), ptr(d["q"]), ptr(d["k"]),
            ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]), ptr(d["state"]), ptr(d["o"]))

    def call():
        st = lib.gdr_decode_step(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(gdr.gdr_status_string(st))
    return call


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy of nbytes (read + write), for context."""
    a = torch.empty(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    _, dt = timed_region(torch, reps, lambda: b.copy_(a))
    del a, b
    return 2 * nbytes * reps / dt / 1e9


def timed_region(torch, steps, body):
    """Synchronize on both sides of exactly `steps` calls to body(); returns
    (wall seconds, GPU seconds between HIP events recorded on the current
    stream -- the stream every launch goes to -- around the region)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        body()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3


def bench_gdn_decode(torch, gdr, synth, steps, warmup, want_cpu):
    w = synth.WORKLOADS["gdn_decode_b64_h32_d128"]
    B, H, dk, dv, L = w.B, w.H, w.dk, w.dv, w.layers
    g = torch.Generator(device="cuda")
    layers = []
    for layer in range(L):
        inp = synth.make_inputs(w, layer=layer, s0="zero")
        g.manual_seed(1000 + layer)
        state = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.02
        d = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, 0])).to(
            torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
            for k in ("q", "k", "v", "alpha", "beta")}
        d["state"] = state
        d["o"] = torch.empty(B, H, dv, device="cuda", dtype=torch.bfloat16)
        layers.append(d)

    calls = [c_decode_call(torch, gdr, "gdn", d) for d in layers]

    def step():
        for c in calls:
            c()

    # One step (48 launches) captured as a HIP graph and replayed: the
    # timed region is GPU work only, with no host launch gaps.
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(2):
        graph.replay()
    elapsed, gpu_s = timed_region(torch, steps, graph.replay)
    launch_ms = 1e3 * gpu_s / (steps * L)
    per_launch = B * H * decode_bytes_per_head("gdn", dk, dv)
    step_bytes = per_launch * L
    res = {
        "elapsed_s": elapsed,
        "ms_per_step": 1e3 * elapsed / steps,
        "gbs": step_bytes * steps / elapsed / 1e9,
        "tokens_per_s": B * steps / elapsed,
        "launch_ms": launch_ms,
        "bytes_per_launch": per_launch,
    }
    if want_cpu:
        res["cpu"] = cpu_baseline_decode(torch, synth, w, layers)
    return res


def cpu_baseline_decode(torch, synth, w, layers, budget_s=12.0):
    """The float64 oracle on whole layers of the same workload until ~budget_s."""
    import oracle
    nt = oracle.default_threads()
    done, t_total = 0, 0.0
    for layer, d in enumerate(layers):
        inp = synth.make_inputs(w, layer=layer, s0="zero")
        s0 = d["state"].double().cpu().numpy()
        x = {k: inp[k][:, 0] for k in ("q", "k", "v", "alpha", "beta")}
        t0 = time.perf_counter()
        oracle.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], s0, nthreads=nt)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    per_layer = w.B * w.H * decode_bytes_per_head("gdn", w.dk, w.dv)
    return {
        "value": round(per_layer * done / t_total / 1e9, 3),
        "unit": "GB/s",
        "cores": nt,
        "kind": "oracle",
        "sample": "%d of %d layers, one decode step each (B=%d, H=%d, d=%d), float64" % (
            done, w.layers, w.B, w.H, w.dk),
        "seconds": round(t_total, 3),
        "cpu": cpu_model(),
    }


def bench_kda_decode(torch, gdr, synth, steps, warmup, want_cpu=False):
    w = synth.WORKLOADS["kda_decode_b256_h32_d128"]
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    inp = synth.make_inputs(w, s0="zero")
    g = torch.Generator(device="cuda")
    g.manual_seed(2000)
    state = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.02
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, 0])).to(
        torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
        for k in ("q", "k", "v", "alpha", "beta")}
    d["state"] = state
    d["o"] = torch.empty(B, H, dv, device="cuda", dtype=torch.bfloat16)
    s_host = state.double().cpu().numpy() if want_cpu else None
    call = c_decode_call(torch, gdr, "kda", d)
    for _ in range(warmup):
        call()
    n = max(steps, 20)
    elapsed, gpu_s = timed_region(torch, n, call)
    launch_ms = 1e3 * gpu_s / n
    per_launch = B * H * decode_bytes_per_head("kda", dk, dv)
    res = {"workload": w.name, "steps": n, "ms_per_step": 1e3 * elapsed / n,
           "gbs": per_launch * n / elapsed / 1e9, "tokens_per_s": B * n / elapsed,
           "roofline": roofline_hbm(per_launch, launch_ms,
                                    load_traffic("decode_kda", src_hash("decode.hip")))}
    if want_cpu:
        import oracle
        x = {k: inp[k][:, 0] for k in ("q", "k", "v", "alpha", "beta")}
        res["cpu_baseline"] = oracle_baseline(
            lambda nt: oracle.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], s_host,
                                          nthreads=nt),
            per_launch / 1e9, "GB/s", "full run: one decode step of all %d heads, float64" % (B * H),
            per_launch / (launch_ms / 1e3) / 1e9)
    return res


def bench_tiny(torch, gdr, synth, steps, warmup, want_cpu=False):
    """The small fp32 GDN case (B=1, H=2, T=64, d=16): one chunked prefill,
    and the same 64 tokens as 64 decode steps.  Latency-bound: times only,
    no roofline fraction."""
    w = synth.WORKLOADS["gdn_tiny_f32"]
    inp = synth.make_inputs(w)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    d = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inp.items()}
    s_out = torch.empty(B, H, dk, dv, device="cuda")
    o = torch.empty(B, T, H, dv, device="cuda")
    pre = lambda: gdr.gdr_chunk_prefill("gdn", d["q"], d["k"], d["v"], d["alpha"], d["beta"], None,
                                        s_out, o)
    steps_in = [{k: d[k][:, t].contiguous() for k in ("q", "k", "v", "alpha", "beta")} for t in range(T)]
    state = torch.zeros(B, H, dk, dv, device="cuda")
    o1 = torch.empty(B, H, dv, device="cuda")
    calls = [c_decode_call(torch, gdr, "gdn", dict(x, state=state, o=o1)) for x in steps_in]

    def dec():
        for c in calls:
            c()
    n = max(steps, 20)
    res = {"workload": w.name, "steps": n}
    for tag, fn in (("prefill", pre), ("decode_x64", dec)):
        for _ in range(warmup):
            fn()
        elapsed, gpu_s = timed_region(torch, n, fn)
        res[tag + "_ms"] = 1e3 * gpu_s / n
        res[tag + "_tokens_per_s"] = B * T * n / elapsed
    res["roofline"] = None
    if want_cpu:
        import oracle
        res["cpu_baseline"] = oracle_baseline(
            lambda nt: oracle.recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None,
                                        nthreads=nt),
            B * T, "tokens/s", "full run (all %d tokens of both heads), float64, mean of 200" % T,
            res["prefill_tokens_per_s"], reps=200)
    return res


def bench_decode_prologue(torch, gdr, synth, steps, warmup, gate="gdn"):
    """The decode step with the fused input prologue (raw q, k normalised and
    gate logits through the sigmoid inside the kernel) beside the plain step,
    same shapes and memory, launches alternating in one region each."""
    import ctypes
    w = synth.WORKLOADS["gdn_decode_b64_h32_d128" if gate == "gdn" else "kda_decode_b256_h32_d128"]
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    lib = gdr.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    g = torch.Generator(device="cuda")
    g.manual_seed(5000)
    args = {}
    # raw inputs for the prologue, the usual (transformed) ones for the plain step
    for f, inp in ((1, synth.make_raw_inputs(w, s0="zero")), (0, synth.make_inputs(w, s0="zero"))):
        d = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, 0])).to(
            torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
            for k in ("q", "k", "v", "alpha", "beta")}
        d["state"] = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.02
        d["o"] = torch.empty(B, H, dv, device="cuda", dtype=torch.bfloat16)
        args[f] = (d, (B, H, dk, dv, ctypes.c_float(1.0), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]),
                       ptr(d["alpha"]), ptr(d["beta"]), ptr(d["state"]), ptr(d["o"])))
    flags = gdr.PRO_L2NORM_QK | gdr.PRO_SIGMOID

    def call(f):
        st = lib.gdr_decode_step_ex(gdr.GATES[gate], 1, f, *args[1 if f else 0][1],
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(gdr.gdr_status_string(st))
    for _ in range(warmup):
        call(flags)
        call(0)
    n = max(steps, 20)
    per_launch = B * H * decode_bytes_per_head(gate, dk, dv)
    res = {"workload": w.name + "_prologue", "steps": n, "bytes_per_launch": per_launch}
    for tag, f in (("prologue", flags), ("plain", 0)):
        _, gpu_s = timed_region(torch, n, lambda: call(f))
        res[tag + "_launch_ms"] = 1e3 * gpu_s / n
    res["overhead"] = round(res["prologue_launch_ms"] / res["plain_launch_ms"] - 1.0, 4)
    res["roofline"] = roofline_hbm(per_launch, res["prologue_launch_ms"], None)
    return res


def bench_gdn_verify(torch, gdr, synth, steps, warmup, T=4, save=True):
    """The verify step of speculative decoding at the decode workload's shape:
    T draft tokens per head in one gdr_decode_multi call, keeping the state
    after every token (for rollback) when ``save``."""
    import ctypes
    w = synth.WORKLOADS["gdn_decode_b64_h32_d128"]
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    inp = synth.make_inputs(w, T=T, s0="zero")
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(
        torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
        for k in ("q", "k", "v", "alpha", "beta")}
    g = torch.Generator(device="cuda")
    g.manual_seed(3000)
    state = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.02
    o = torch.empty(B, T, H, dv, device="cuda", dtype=torch.bfloat16)
    states = torch.empty(B, T, H, dk, dv, device="cuda") if save else None
    lib = gdr.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    args = (gdr.GATES["gdn"], 1, B, T, H, dk, dv, ctypes.c_float(1.0), ptr(d["q"]), ptr(d["k"]),
            ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]), ptr(state), ptr(o), ptr(states))

    def call():
        st = lib.gdr_decode_multi(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(gdr.gdr_status_string(st))
    for _ in range(warmup):
        call()
    n = max(steps, 20)
    elapsed, gpu_s = timed_region(torch, n, call)
    launch_ms = 1e3 * gpu_s / n
    per_launch = B * H * verify_bytes_per_head("gdn", dk, dv, T, save)
    return {"workload": "gdn_verify_b64_h32_d128_t%d%s" % (T, "" if save else "_nostates"),
            "steps": n, "ms_per_step": 1e3 * elapsed / n, "launch_ms": launch_ms,
            "tokens_per_s": B * T * n / elapsed, "gbs": per_launch * n / elapsed / 1e9,
            "bytes_per_launch": per_launch,
            "roofline": roofline_hbm(per_launch, launch_ms,
                                     load_traffic("verify_gdn" + ("" if save else "_nostates"),
                                                  src_hash("decode.hip")))}


def varlen_lengths(N=32, lo=128, hi=4096, seed=7):
    """Prompt lengths of the packed variable-length workload (seeded, log-uniform)."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(np.log(lo), np.log(hi), N)).astype(np.int64).tolist()


def bench_gdn_varlen(torch, gdr, synth, steps, warmup, N=32, slots=64):
    """Packed variable-length GDN prefill of N prompts (a serving batch): every
    prompt reads its state from a pooled row and writes it back."""
    w = synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128"]
    H, dk, dv = w.H, w.dk, w.dv
    lens = varlen_lengths(N)
    total = int(sum(lens))
    inp = synth.make_inputs(w, B=1, T=total, s0="zero")
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k][0])).to(
        torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
        for k in ("q", "k", "v", "alpha", "beta")}
    del inp
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    perm = np.random.default_rng(11).permutation(slots)[:N]
    sl = torch.tensor(perm, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(4000)
    pool = torch.randn(slots, H, dk, dv, device="cuda", generator=g) * 0.02
    o = torch.empty(total, H, dv, device="cuda", dtype=torch.bfloat16)
    max_t = int(max(lens))
    need = gdr.gdr_chunk_prefill_varlen_workspace_bytes("gdn", torch.bfloat16, N, max_t, H, dk, dv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    call = lambda: gdr.gdr_chunk_prefill_varlen("gdn", d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                cu, sl, pool, o, max_seqlen=max_t, workspace=ws)
    for _ in range(warmup):
        call()
    n = max(5, steps // 2)
    elapsed, gpu_s = timed_region(torch, n, call)
    launch_ms = 1e3 * gpu_s / n
    # every token's q, k, v, o and gates, and each prompt's state read and written once
    per_launch = prefill_bytes("gdn", 1, total, H, dk, dv, False) - H * 4 * dk * dv + 2 * N * H * 4 * dk * dv
    return {"workload": "gdn_prefill_varlen_n%d_h%d_d%d" % (N, H, dk), "steps": n,
            "ms_per_step": 1e3 * elapsed / n, "launch_ms": launch_ms,
            "tokens_per_s": total * n / elapsed, "tokens": total, "lengths": "%d prompts, %d..%d tokens" % (N, min(lens), max(lens)),
            "algorithmic_bytes": per_launch,
            "roofline": roofline_hbm(per_launch, launch_ms, None)}


def backward_flops(B, T, H, dk, dv):
    """Flops of the chunked backward as computed (per 64-token chunk and
    head; a fused multiply-add counts 2): the chunk-local prep (Ahat, P over
    the lower triangle, the triangular inverse), the forward checkpoint chain
    (Xr, U, S), the reverse chain (U, dU, dX, dS) and the chunk-local
    contractions (dQ0, dK0, dKt, dA, dP and the four gate-weighted sums)."""
    C, tri = CHUNK, CHUNK * (CHUNK + 1) // 2
    per = (2 * tri * dk * 2 + C ** 3 // 3 * 2                          # prep
           + (C * dk * dv + tri * dv + dk * C * dv) * 2                # forward chain
           + (tri * dv + tri * dv + C * dk * dv + tri * dv + 2 * C * dk * dv) * 2  # reverse chain
           + (3 * C * dk * dv + 2 * C * C * dv + 4 * tri * dk) * 2)    # local
    nch = (T + CHUNK - 1) // CHUNK
    return B * H * nch * per


def backward_bytes(gate, B, T, H, dk, dv, elt=2):
    """Algorithmic HBM bytes: read q, k, v, dO and the gates, write dq, dk, dv
    and the gate gradients; read S_0 and dS_T, write dS_0."""
    g = 4 * dk if gate == "kda" else 4
    per_tok = elt * (2 * dk + 2 * dv) + g + 4 + elt * (2 * dk + dv) + g + 4
    return B * T * H * per_tok + 3 * B * H * 4 * dk * dv


def bench_backward(torch, gdr, synth, name, steps, warmup):
    """One gdr_chunk_backward per step on the prefill workload's shape (bf16
    inputs and output gradient, fp32 state and state gradient)."""
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    d = {k: torch.from_numpy(v).to(torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()
         for k, v in inp.items() if v is not None}
    del inp
    g = torch.Generator(device="cuda")
    g.manual_seed(6000)
    do = torch.randn(B, T, H, dv, device="cuda", generator=g).to(torch.bfloat16)
    dst = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.1
    s0 = d.get("s0")
    out = [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
           torch.empty_like(d["alpha"]), torch.empty_like(d["beta"]),
           torch.empty(B, H, dk, dv, device="cuda")]
    need = gdr.gdr_chunk_backward_workspace_bytes(w.gate, torch.bfloat16, B, T, H, dk, dv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    call = lambda: gdr.gdr_chunk_backward(w.gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, do,
                                          dst, *out, workspace=ws)
    for _ in range(warmup):
        call()
    elapsed, gpu_s = timed_region(torch, steps, call)
    launch_ms = 1e3 * gpu_s / steps
    # the same in chunk ranges, with a workspace of at most 2 GB
    nch = (T + CHUNK - 1) // CHUNK
    rc = next((c for c in range(nch - 1, 0, -1)
               if gdr.gdr_chunk_backward_workspace_bytes_ranged(w.gate, torch.bfloat16, B, T, H, dk, dv, c)
               <= 2 * 10 ** 9), 1)
    need_r = gdr.gdr_chunk_backward_workspace_bytes_ranged(w.gate, torch.bfloat16, B, T, H, dk, dv, rc)
    del ws
    ws_r = torch.empty(need_r, dtype=torch.uint8, device="cuda")
    call_r = lambda: gdr.gdr_chunk_backward(w.gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, do,
                                            dst, *out, workspace=ws_r)
    call_r()
    _, gpu_r = timed_region(torch, steps, call_r)
    flops = backward_flops(B, T, H, dk, dv)
    nbytes = backward_bytes(w.gate, B, T, H, dk, dv)
    sec = launch_ms / 1e3
    return {"workload": name.replace("prefill", "backward"), "steps": steps,
            "ms_per_step": 1e3 * elapsed / steps, "launch_ms": launch_ms,
            "tokens_per_s": B * T * steps / elapsed, "workspace_bytes": need,
            "ranged": {"range_chunks": rc, "workspace_bytes": need_r, "launch_ms": 1e3 * gpu_r / steps},
            "roofline": {"bound": "alu", "achieved": round(flops / sec / 1e12, 2), "peak": FP32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(flops / sec / 1e12 / FP32_PEAK_TFLOPS, 4),
                         "traffic": load_traffic("backward_" + w.gate, src_hash("backward.hip")),
                         "algorithmic_flops": flops},
            "hbm": {"achieved": round(nbytes / sec / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}}


def bench_prefill(torch, gdr, synth, name, steps, warmup, flags=0, want_cpu=False):
    """One chunked prefill per step; with ``flags`` the inputs are raw (q, k
    not normalised, gate logits) and the kernels run the input prologue.
    ``want_cpu``: the float64 oracle runs the whole workload on the same
    inputs afterwards."""
    w = synth.WORKLOADS[name]
    inp = synth.make_raw_inputs(w) if flags else synth.make_inputs(w)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    d = {k: (None if v is None else torch.from_numpy(v).to(
        torch.bfloat16 if k in ("q", "k", "v") else torch.float32).cuda()) for k, v in inp.items()}
    if not want_cpu:
        del inp
    s_out = torch.empty(B, H, dk, dv, device="cuda")
    o = torch.empty(B, T, H, dv, device="cuda", dtype=torch.bfloat16)
    need = gdr.gdr_chunk_prefill_workspace_bytes(w.gate, torch.bfloat16, B, T, H, dk, dv, flags=flags)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    call = lambda: gdr.gdr_chunk_prefill_ex(w.gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                            d["s0"], s_out, o, flags=flags, workspace=ws)
    for _ in range(warmup):
        call()
    elapsed, gpu_s = timed_region(torch, steps, call)
    launch_ms = 1e3 * gpu_s / steps
    nbytes = prefill_bytes(w.gate, B, T, H, dk, dv, d["s0"] is not None)
    flops = prefill_flops(B, T, H, dk, dv)
    sec = launch_ms / 1e3
    cpu = None
    if want_cpu:
        import oracle
        cpu = oracle_baseline(
            lambda nt: oracle.recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"],
                                        nthreads=nt),
            B * T, "tokens/s", "full run (all %d heads, %d tokens each), float64" % (B * H, T),
            B * T / sec)
        del inp
    res = {
        "workload": name + ("_prologue" if flags else ""), "steps": steps,
        "ms_per_step": 1e3 * elapsed / steps,
        "tokens_per_s": B * T * steps / elapsed,
        "schedule": "split" if need else "fused", "workspace_bytes": need,
        "launch_ms": launch_ms,
        "roofline": {
            "bound": "hbm", "achieved": round(nbytes / sec / 1e9, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None if flags else load_traffic("prefill_" + w.gate, src_hash("prefill_bf16.hip")),
        },
        "mfma": {"achieved": round(flops / sec / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "algorithmic_flops": flops},
        "algorithmic_bytes": nbytes,
    }
    if cpu:
        res["cpu_baseline"] = cpu
    return res


def roofline_hbm(per_launch_bytes, launch_ms, traffic=None):
    a = per_launch_bytes / (launch_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default=None,
                    help="gdn_decode | kda_decode | tiny | gdn_verify | gdn_prefill | gdn_varlen | kda_prefill | "
                         "backward | prologue | copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_08_amd as gdr
    import synth
    if not os.path.exists(gdr.library_path()):
        from gated_delta_rule_08_amd import build
        build.build()
    gdr.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)

    only = args.only
    if only == "copy":  # plain copy kernel of known size, for counter calibration
        print(json.dumps({"copy_gbs_measured": round(copy_bandwidth(torch), 1),
                          "bytes_per_copy": 1 << 30}))
        return
    extra = {}
    head = None
    if only in (None, "gdn_decode"):
        head = bench_gdn_decode(torch, gdr, synth, args.steps, args.warmup,
                                want_cpu=(only is None and not args.no_cpu_baseline))
    want_cpu = only is None and not args.no_cpu_baseline
    if only in (None, "kda_decode"):
        extra["kda_decode_b256_h32_d128"] = bench_kda_decode(torch, gdr, synth, args.steps,
                                                             args.warmup, want_cpu)
    if only in (None, "tiny"):
        extra["gdn_tiny_f32"] = bench_tiny(torch, gdr, synth, args.steps, args.warmup, want_cpu)
    if only in (None, "gdn_verify"):
        for save in (True, False):
            r = bench_gdn_verify(torch, gdr, synth, args.steps, args.warmup, T=4, save=save)
            extra[r["workload"]] = r
    if only in (None, "gdn_prefill"):
        extra["gdn_prefill_b4_t8192_h32_d128"] = bench_prefill(
            torch, gdr, synth, "gdn_prefill_b4_t8192_h32_d128", max(5, args.steps // 2), 2,
            want_cpu=want_cpu)
    if only in (None, "gdn_varlen"):
        r = bench_gdn_varlen(torch, gdr, synth, args.steps, 2)
        extra[r["workload"]] = r
    if only in (None, "kda_prefill"):
        extra["kda_prefill_b1_t32768_h32_d128"] = bench_prefill(
            torch, gdr, synth, "kda_prefill_b1_t32768_h32_d128", max(5, args.steps // 2), 2,
            want_cpu=want_cpu)
    if only in (None, "backward"):
        for name in ("gdn_prefill_b4_t8192_h32_d128", "kda_prefill_b1_t32768_h32_d128"):
            r = bench_backward(torch, gdr, synth, name, max(3, args.steps // 4), 1)
            extra[r["workload"]] = r
    if only in (None, "prologue"):  # the same paths with the fused input prologue
        for gate in ("gdn", "kda"):
            r = bench_decode_prologue(torch, gdr, synth, args.steps, args.warmup, gate)
            extra[r["workload"]] = r
        pro = gdr.PRO_L2NORM_QK | gdr.PRO_SIGMOID
        for name in ("gdn_prefill_b4_t8192_h32_d128", "kda_prefill_b1_t32768_h32_d128"):
            r = bench_prefill(torch, gdr, synth, name, max(5, args.steps // 2), 2, flags=pro)
            extra[r["workload"]] = r

    if head is None:
        print(json.dumps({"workloads": extra}))
        return
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gdn_decode_b64_h32_d128", "gate": "gdn", "B": 64, "H": 32,
                   "dk": 128, "dv": 128, "layers": 48, "qkv": "bf16", "state": "fp32",
                   "tokens_per_s": round(head["tokens_per_s"], 1)},
        "roofline": roofline_hbm(head["bytes_per_launch"], head["launch_ms"],
                                 load_traffic("decode_gdn", src_hash("decode.hip"))),
    }
    if "cpu" in head:
        line["cpu_baseline"] = head["cpu"]
    line["context"] = {"copy_gbs_measured": round(copy_bandwidth(torch), 1),
                       "note": "device-to-device copy of 1 GiB on the same GPU, same run"}
    if extra:
        line["workloads"] = extra
    print(json.dumps(line))


if __name__ == "__main__":
    main()
