#!/usr/bin/env python3
"""Throughput of the fused MoE layer forward on one MI355X.

One step = one whole layer call (router + dispatch, expert gate/up, expert
down + weighted combine) through the C ABI on one batch of synthetic inputs
already resident in HBM.  Weight sets are rotated between steps so that every
step streams its weights from HBM rather than from the 256 MB Infinity Cache.

With no --workload the run covers the whole metric: the headline record is
the Mixtral-8x7B-shaped decode layer at T=8 (hidden 4096, 8 experts, top-2,
SwiGLU intermediate 14336, bf16 weights), and the same JSON line nests the
records of the 256-expert Q4_0 decode at T=1 (top-8 + 1 shared expert), the
DeepSeek-MoE-16B-shaped decode at T=8 and T=64, and the Mixtral-shaped
4096-token prefill with Zipf routing.  --workload NAME times one workload.

Prints ONE JSON line on stdout.  Each record carries
  value, ms_per_step  tokens/s and time of exactly --steps timed steps;
  spread        median / p10 / p90 of ms per step over 5 repetitions of the
                timed loop;
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                divided by its average launch duration, measured with HIP
                events recorded on the launch stream around that kernel, with
                frac against the published peak and frac_measured against
                the probes below;
  layer         the same for the whole layer: algorithmic bytes (or flops)
                of one call over ms_per_step;
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample,
                with all BLAS threads and with one.
The headline line also carries `probes`: a cold streaming read of >= 1 GiB
and the bandwidth-versus-bytes curve of one read kernel (including the
Q4_0 layer's 18 MB), and back-to-back bf16 MFMAs on every compute unit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MoE-layer tokens/s at decode bs=1/8 (HBM GB/s %) and prefill 4096 (MFMA %)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
COLD_BYTES = 10 * 2 ** 30       # rotate weight copies until ~40x the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ HIP events ----

class HipEvents:
    """Minimal ctypes access to hipEvent_* (the library torch already loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0)
            if rc:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            evs.append(e.value)
        return evs

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


# ---------------------------------------------------------- byte counting ----

def mat_bytes(w_dtype, N, K):
    """Stored bytes of one weight matrix [N, K], scales included."""
    if w_dtype == "f32":
        return 4 * N * K
    if w_dtype == "bf16":
        return 2 * N * K
    if w_dtype == "q4_0":
        return N * K // 2 + 2 * N * (K // 32)
    if w_dtype == "q8_0":
        return N * K + 2 * N * (K // 32)
    if w_dtype == "fp8_e4m3":
        return N * K + 4 * N
    raise ValueError(w_dtype)


def act_bytes(dt):
    return 4 if dt == "f32" else 2


def h_elem_bytes(wl):
    """Bytes per element of the activation rows between the decode launches."""
    return 4 if wl.w_dtype in ("f32", "bf16") else 2


def layer_bytes(wl):
    """Bytes of one full copy of the layer's weights (all experts)."""
    return (wl.E * (2 * mat_bytes(wl.w_dtype, wl.I, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.I))
            + wl.S * (2 * mat_bytes(wl.w_dtype, wl.Is, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.Is))
            + wl.E * wl.H * act_bytes(wl.r_dtype))


def gateup_alg_bytes(wl, n_active, T, shared=True):
    """Algorithmic bytes of one decode gate/up launch: the engaged experts' gate
    and up rows, the activations read and the intermediate rows written (the
    shared experts' part only when the launch computes them: with
    shared=False they run in the router launch)."""
    S = wl.S if shared else 0
    return (n_active * 2 * mat_bytes(wl.w_dtype, wl.I, wl.H) + S * 2 * mat_bytes(wl.w_dtype, wl.Is, wl.H)
            + T * wl.H * act_bytes(wl.x_dtype) + (T * wl.k * wl.I + S * T * wl.Is) * h_elem_bytes(wl))


def down_alg_bytes(wl, n_active, T):
    return (n_active * mat_bytes(wl.w_dtype, wl.H, wl.I) + wl.S * mat_bytes(wl.w_dtype, wl.H, wl.Is)
            + (T * wl.k * wl.I + wl.S * T * wl.Is) * h_elem_bytes(wl) + T * wl.H * act_bytes(wl.x_dtype))


def layer_alg_bytes(wl, n_active, T):
    return (n_active * (2 * mat_bytes(wl.w_dtype, wl.I, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.I))
            + wl.S * (2 * mat_bytes(wl.w_dtype, wl.Is, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.Is))
            + wl.E * wl.H * act_bytes(wl.r_dtype) + T * wl.H * 2 * act_bytes(wl.x_dtype))


def sparse_layer_alg_bytes(wl, T):
    """Channel-sparse layer: the kept rows of gate, up and (transposed) down of
    each engaged expert, the routed experts' channel scores, the dense shared
    experts, the router, and x / out."""
    import synth
    c = synth.channel_count(wl)
    row = mat_bytes(wl.w_dtype, 1, wl.H)
    return (T * wl.k * (3 * c * row + wl.I * 4)
            + wl.S * (2 * mat_bytes(wl.w_dtype, wl.Is, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.Is))
            + wl.E * wl.H * act_bytes(wl.r_dtype) + T * wl.H * 2 * act_bytes(wl.x_dtype))


def gateup_flops(wl):
    return 2.0 * (wl.T * wl.k * 2 * wl.I * wl.H + wl.T * wl.S * 2 * wl.Is * wl.H)


def layer_flops(wl):
    return 2.0 * (wl.T * wl.k * 3 * wl.I * wl.H + wl.T * wl.S * 3 * wl.Is * wl.H + wl.T * wl.H * wl.E)


def kernel_source_hash():
    """Hash of everything that decides what the kernels do and how they are
    launched: every source of the library (kernels, launch code, path and grid
    choice in api.cpp) and the compiler flags."""
    from mixture_experts_layer_12_amd import build as b
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_12_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    h.update(" ".join(b.FLAGS).encode())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM traffic per launch from committed rocprofv3 counter summaries, only
    when they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------- CPU oracle ----

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, t, tokens_max=16, min_seconds=5.0):
    """The fp64 oracle on a bounded sample of the same workload: the first
    min(T, tokens_max) tokens of weight copy 0, decoding from the stored bits
    only the experts those tokens reach.  Repeated for at least min_seconds
    with every BLAS thread, then once with one thread."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    n_tok = min(wl.T, tokens_max)

    def f64(a):
        if a.dtype == torch.bfloat16:
            return oracle.bf16_to_f64(a.cpu().view(torch.int16).numpy().view(np.uint16))
        return a.cpu().numpy().astype(np.float64)

    def mat(key, e, n_mat, N, K):
        a = t[key]
        if wl.w_dtype == "q4_0":
            return oracle.q4_0_decode_matrix(a.cpu().numpy(), n_mat, N, K, e)
        if wl.w_dtype in ("q8_0", "fp8_e4m3"):
            off = (n_mat * N * K + 255) // 256 * 256          # scales after all one-byte codes
            codes = a[e * N * K:(e + 1) * N * K].cpu().numpy().reshape(N, K)
            if wl.w_dtype == "q8_0":
                nb = N * (K // 32) * 2
                return oracle.q8_0_matrix(codes, a[off + e * nb:off + (e + 1) * nb].cpu().numpy().view(np.uint16)
                                          .reshape(N, K // 32))
            return oracle.fp8_e4m3_matrix(codes, a[off + 4 * e * N:off + 4 * (e + 1) * N].cpu().numpy()
                                          .view(np.float32))
        return f64(a[e])

    def once():
        x = f64(t["x"][:n_tok])
        Wr = f64(t["router_w"])
        b = None if t["router_b"] is None else f64(t["router_b"])
        l, p, ids, w = oracle.route(x, Wr, b, wl.k)
        out = np.zeros((n_tok, wl.H))
        for e in np.unique(ids):
            rows, js = np.nonzero(ids == e)
            y = oracle.swiglu_ffn(x[rows], mat("w_gate", e, wl.E, wl.I, wl.H), mat("w_up", e, wl.E, wl.I, wl.H),
                                  mat("w_down", e, wl.E, wl.H, wl.I))
            np.add.at(out, rows, w[rows, js][:, None] * y)
        for s in range(wl.S):
            out += oracle.swiglu_ffn(x, mat("ws_gate", s, wl.S, wl.Is, wl.H), mat("ws_up", s, wl.S, wl.Is, wl.H),
                                     mat("ws_down", s, wl.S, wl.H, wl.Is))
        return out

    reps, t0 = 0, time.perf_counter()
    while True:
        once()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el > 0 and reps >= 50:
            break
    threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        once()
        el1 = time.perf_counter() - t1
    return {"value": reps * n_tok / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tok} of {wl.T} tokens of one layer call (weight copy 0), x{reps} repetitions, "
                      f"fp64 numpy oracle including decoding the stored weights of the experts those tokens reach; "
                      f"{el:.1f} s",
            "value_1_thread": n_tok / el1, "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


# ------------------------------------------------------- channel-sparse -----

def bench_sparse(args, m, wl, inp, copies, dev):
    """The budgeted channel-sparse layer (moe_forward_channel_sparse): per-copy
    channel scores and transposed down stacks, whole-layer timing."""
    import torch
    c = synth.channel_count(wl)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 1)
    scores = [torch.randn((wl.T, wl.E, wl.I), generator=gen, device=dev) for _ in range(copies)]
    wdt = [w.transpose(1, 2).contiguous() for w in inp["w_down"]]
    shape = m.make_shape(wl.T, wl.H, wl.E, wl.I, wl.k, wl.S, wl.Is, wl.x_dtype, wl.w_dtype, wl.r_dtype)
    ws = m.alloc_sparse_workspace(shape, c, dev)
    out = torch.empty_like(inp["x"][0])
    sh = torch.cuda.current_stream().cuda_stream

    def step(i):
        j = i % copies
        m.moe_forward_channel_sparse(shape, c, scores[j], inp["x"][j], inp["router_w"][j], inp["router_b"][j],
                                     inp["w_gate"][j], inp["w_up"][j], wdt[j], inp["ws_gate"][j], inp["ws_up"][j],
                                     inp["ws_down"][j], out, ws, stream=sh)

    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed
    alg = sparse_layer_alg_bytes(wl, wl.T)
    achieved = alg / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] sparse c={c} of I={wl.I}: {ms_per_step * 1e3:.1f} us/step, {value:.1f} tokens/s, {achieved:.0f} GB/s")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "layer (all launches of one call)",
            "launch_ms": round(ms_per_step, 5), "alg_bytes_per_launch": int(alg), "channels_kept": c}
    cpu = None
    if not args.no_cpu:
        import numpy as np
        import oracle
        x = inp["x"][0].float().cpu().numpy().astype(np.float64)
        Wr = inp["router_w"][0].float().cpu().numpy().astype(np.float64)
        sc = scores[0].cpu().numpy().astype(np.float64)
        t_start = time.perf_counter()
        n = 0
        while True:
            l, p, ids, w = oracle.route(x, Wr, None, wl.k)
            for t in range(wl.T):
                for j in range(wl.k):
                    e = int(ids[t, j])
                    Wg = inp["w_gate"][0][e].float().cpu().numpy().astype(np.float64)
                    Wu = inp["w_up"][0][e].float().cpu().numpy().astype(np.float64)
                    Wd = inp["w_down"][0][e].float().cpu().numpy().astype(np.float64)
                    oracle.masked_swiglu(x[t:t + 1], Wg, Wu, Wd, oracle.select_channels(sc[t, e], c))
            n += 1
            if time.perf_counter() - t_start > 5.0:
                break
        el = time.perf_counter() - t_start
        cpu = {"value": wl.T * n / el, "unit": "tokens/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{n} calls of the whole batch ({wl.T} token(s)), fp64 numpy oracle including decoding the "
                         f"engaged experts' weights; {el:.1f} s"}
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.w_dtype, "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "top_k": wl.k, "I": wl.I,
                   "n_shared": wl.S, "I_shared": wl.Is, "weights": wl.w_dtype, "activations": wl.x_dtype,
                   "router": wl.r_dtype, "path": "channel_sparse", "channels_kept": c, "weight_copies": copies,
                   "timing": "eager launches", "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    return rec


# ---------------------------------------------------------------- probes ----

PROBE_SIZES_MB = [1, 2, 4, 8, 16, 18.04, 32, 64, 128, 256, 512, 1024, 4096]


def run_probes(m, dev, hip):
    """Measured peaks: a cold streaming read (median over distinct >= 1 GiB
    regions), the bandwidth of one read kernel against the bytes it reads (each
    size read at distinct offsets of an 8 GiB buffer, so every read is cold),
    and bf16 MFMA throughput on register operands."""
    import torch
    total = 8 * 2 ** 30
    buf = torch.zeros(total, dtype=torch.uint8, device=dev)
    sink = torch.empty(2 ** 20, dtype=torch.uint8, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    curve = []
    off = 0
    for mb in PROBE_SIZES_MB:
        nbytes = int(mb * 1e6) // 4096 * 4096 if mb != int(mb) else int(mb) * 2 ** 20
        reps = max(2, min(20, total // nbytes))
        gbs = []
        for r in range(reps):
            if off + nbytes > total:
                off = 0
            evs = hip.create(2)
            torch.cuda.synchronize()
            hip.record(evs[0], sh)
            m.moe_probe_read(buf.data_ptr() + off, nbytes, sink, stream=sh)
            hip.record(evs[1], sh)
            torch.cuda.synchronize()
            ms = hip.elapsed_ms(evs[0], evs[1])
            hip.destroy(evs)
            gbs.append(nbytes / (ms * 1e-3) / 1e9)
            off += nbytes
        gbs.sort()
        curve.append({"bytes": nbytes, "gbs_median": round(gbs[len(gbs) // 2], 1), "gbs_max": round(gbs[-1], 1),
                      "reads": reps})
        log(f"[probe] read {nbytes / 1e6:9.2f} MB: median {gbs[len(gbs) // 2]:7.1f} GB/s")
    big = [c["gbs_median"] for c in curve if c["bytes"] >= 2 ** 30]
    stream_peak = max(big)
    del buf
    # MFMA: about 5 ms per launch, best of 3
    iters = 40000
    best = 0.0
    for _ in range(3):
        evs = hip.create(2)
        torch.cuda.synchronize()
        hip.record(evs[0], sh)
        fl = m.moe_probe_mfma_bf16(iters, sink, stream=sh)
        hip.record(evs[1], sh)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(evs[0], evs[1])
        hip.destroy(evs)
        best = max(best, fl / (ms * 1e-3) / 1e12)
    log(f"[probe] cold streaming read {stream_peak:.1f} GB/s; bf16 MFMA {best:.1f} TFLOP/s")
    torch.cuda.empty_cache()
    return {"stream_read_gbs": stream_peak, "mfma_bf16_tflops": round(best, 1), "read_curve": curve,
            "command": "bench.py probes: moe_probe_read / moe_probe_mfma_bf16 (include/moe_probe.h)"}


def curve_at(probes, nbytes):
    """Measured read bandwidth of one kernel reading about nbytes (nearest curve point)."""
    if not probes:
        return None
    c = min(probes["read_curve"], key=lambda p: abs(math.log(p["bytes"] / nbytes)))
    return c["gbs_median"]


# --------------------------------------------------------------- measure ----

def measure(args, m, wl, dev, hip, probes=None, cpu_seconds=5.0):
    """One workload: its record (value, spread, roofline, layer, cpu_baseline)."""
    import torch
    copies = args.copies or max(1, min(32, math.ceil(COLD_BYTES / layer_bytes(wl))))
    log(f"[bench] workload {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.S} Is={wl.Is} "
        f"w={wl.w_dtype} x={wl.x_dtype}; {copies} weight copies of {layer_bytes(wl) / 1e9:.2f} GB")
    inp = synth.make_inputs_torch(wl, args.seed, device=dev, copies=copies)
    if copies == 1:
        inp = {k: [v] for k, v in inp.items()}
    if wl.channel_budget is not None:
        return bench_sparse(args, m, wl, inp, copies, dev)
    path_arg = {"auto": m.MOE_PATH_AUTO, "decode": m.MOE_PATH_DECODE, "fused": m.MOE_PATH_DECODE_FUSED,
                "prefill": m.MOE_PATH_PREFILL}[args.path]
    shape = m.make_shape(wl.T, wl.H, wl.E, wl.I, wl.k, wl.S, wl.Is, wl.x_dtype, wl.w_dtype, wl.r_dtype, path_arg)
    path = m.moe_resolve_path(shape)
    path_name = {m.MOE_PATH_DECODE: "decode", m.MOE_PATH_PREFILL: "prefill",
                 m.MOE_PATH_DECODE_FUSED: "decode_fused"}[path]
    if args.graph and path == m.MOE_PATH_DECODE_FUSED:
        path_name = "decode"       # a captured single-launch decode records the multi-launch form
    ws = m.alloc_workspace(shape, dev)
    out = torch.empty_like(inp["x"][0])
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(i, events=None):
        c = i % copies
        a = (shape, inp["x"][c], inp["router_w"][c], inp["router_b"][c], inp["w_gate"][c], inp["w_up"][c],
             inp["w_down"][c], inp["ws_gate"][c], inp["ws_up"][c], inp["ws_down"][c], out, ws)
        if events is None:
            m.moe_forward(*a, stream=sh)
        else:
            m.moe_forward_profiled(*a, events, stream=sh)

    def timed(fn, n, first):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(first + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # residency: one untimed call per weight copy, so that no timed step is the
    # first GPU access to a buffer (page-table set-up is not part of a step)
    torch.cuda.synchronize()
    for c in range(copies):
        step(c)
    # eager warm-up (also performs the library's one-time set-up before any capture)
    torch.cuda.synchronize()
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    if not args.graph:
        fn = step
        timing = "eager launches"
    else:
        # one captured graph per weight copy, replayed in rotation: every replay
        # runs the whole layer (router, dispatch, experts, combine) again
        cap = torch.cuda.Stream()
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                a = (shape, inp["x"][c], inp["router_w"][c], inp["router_b"][c], inp["w_gate"][c], inp["w_up"][c],
                     inp["w_down"][c], inp["ws_gate"][c], inp["ws_up"][c], inp["ws_down"][c], out, ws)
                m.moe_forward(*a, stream=cap.cuda_stream)
            graphs.append(g)
        fn = lambda i: graphs[i % copies].replay()
        for i in range(args.warmup):
            fn(i)
        timing = "hipGraph replay, one graph per weight copy"
    elapsed = timed(fn, args.steps, args.warmup)
    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed
    # spread: the same timed loop repeated
    reps = [ms_per_step] + [timed(fn, args.steps, args.warmup + r * args.steps) * 1e3 / args.steps
                            for r in range(1, args.reps)]
    srt = sorted(reps)

    def pct(q):
        return srt[min(len(srt) - 1, max(0, int(round(q * (len(srt) - 1)))))]
    spread = {"reps": len(reps), "median_ms": round(pct(0.5), 5), "p10_ms": round(pct(0.1), 5),
              "p90_ms": round(pct(0.9), 5), "ms": [round(v, 5) for v in reps]}
    log(f"[bench] {wl.name}: {ms_per_step * 1e3:.1f} us/step, {value:.1f} tokens/s ({timing}); "
        f"reps median {spread['median_ms'] * 1e3:.1f} us, p10 {spread['p10_ms'] * 1e3:.1f}, "
        f"p90 {spread['p90_ms'] * 1e3:.1f}")

    # stage timing with HIP events recorded on the launch stream
    prefill = path_name == "prefill"
    fused = path_name == "decode_fused"
    n_ev = 5 if prefill else (2 if fused else 4)
    evs = [hip.create(n_ev) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    stage = [[hip.elapsed_ms(e[j], e[j + 1]) for j in range(n_ev - 1)] for e in evs]
    for e in evs:
        hip.destroy(e)
    avg = [sum(s_[j] for s_ in stage) / len(stage) for j in range(n_ev - 1)]
    names = (["router", "prefill_gateup", "prefill_down", "combine"] if prefill
             else (["decode_fused"] if fused else ["router", "decode_gateup", "decode_down"]))
    log("[bench] stage averages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in zip(names, avg)))

    # isolated calls: the stream idle before each one (synchronised), the next
    # weight copy (cold), HIP events around the single call -- what one layer
    # costs when nothing is queued behind or ahead of it
    n_iso = min(10, max(2, copies))
    iso_ev = hip.create(2 * n_iso)
    for i in range(n_iso):
        torch.cuda.synchronize()
        hip.record(iso_ev[2 * i], sh)
        step(args.warmup + args.steps + i)
        hip.record(iso_ev[2 * i + 1], sh)
    torch.cuda.synchronize()
    iso = sorted(hip.elapsed_ms(iso_ev[2 * i], iso_ev[2 * i + 1]) for i in range(n_iso))
    hip.destroy(iso_ev)
    isolated = {"calls": n_iso, "median_ms": round(iso[len(iso) // 2], 5), "min_ms": round(iso[0], 5),
                "max_ms": round(iso[-1], 5)}
    log(f"[bench] isolated cold calls: median {isolated['median_ms'] * 1e3:.1f} us "
        f"(min {isolated['min_ms'] * 1e3:.1f}, max {isolated['max_ms'] * 1e3:.1f})")

    # engaged experts per weight copy (from the run's own routing)
    n_active = []
    rws = torch.empty(m.moe_route_workspace_size(shape), dtype=torch.uint8, device=dev)
    for c in range(copies):
        r_out = dict(topk_ids=torch.empty(wl.T * wl.k, dtype=torch.int32, device=dev),
                     topk_w=torch.empty(wl.T * wl.k, dtype=torch.float32, device=dev),
                     active=torch.empty(wl.E + 1, dtype=torch.int32, device=dev))
        m.moe_route(shape, inp["x"][c], inp["router_w"][c], inp["router_b"][c], r_out, rws, stream=sh)
        torch.cuda.synchronize()
        n_active.append(int(r_out["active"][0].item()))
    steps_copies = [(args.warmup + i) % copies for i in range(args.steps)]
    mean_active = sum(n_active[c] for c in steps_copies) / args.steps
    stream_peak = probes["stream_read_gbs"] if probes else None
    mfma_peak = probes["mfma_bf16_tflops"] if probes else None

    def fmeas(a, peak):
        return None if not peak else round(a / peak, 4)

    stages = {n: round(v, 5) for n, v in zip(names, avg)}
    if prefill:
        kname = "prefill_gateup"
        fl = gateup_flops(wl)
        achieved = fl / (avg[1] * 1e-3) / 1e12
        lay = layer_flops(wl) / (ms_per_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(wl.name, kname),
                "kernel": kname, "launch_ms": round(avg[1], 5), "alg_flops_per_launch": fl,
                "frac_measured": fmeas(achieved, mfma_peak)}
        down_fl = layer_flops(wl) - fl - 2.0 * wl.T * wl.H * wl.E
        layer = {"bound": "mfma", "achieved": round(lay, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(lay / MFMA_BF16_PEAK_TFLOPS, 4), "frac_measured": fmeas(lay, mfma_peak),
                 "alg_flops_per_call": layer_flops(wl), "stage_ms": stages,
                 "down_tflops": round(down_fl / (avg[2] * 1e-3) / 1e12, 2)}
    else:
        lay_b = sum(layer_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
        lay = lay_b / (ms_per_step * 1e-3) / 1e9
        if fused:
            kname = "decode_fused"
            alg = lay_b
            achieved = alg / (avg[0] * 1e-3) / 1e9
            klaunch = avg[0]
        else:
            kname = "decode_gateup"
            # with the shared experts' gate/up in the router launch, the routed gate/up launch reads no shared rows
            shared_here = not m.moe_forward_tables(shape)["shared_in_router"]
            alg = sum(gateup_alg_bytes(wl, n_active[c], wl.T, shared_here) for c in steps_copies) / args.steps
            achieved = alg / (avg[1] * 1e-3) / 1e9
            klaunch = avg[1]
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name, kname),
                "kernel": kname, "launch_ms": round(klaunch, 5), "alg_bytes_per_launch": int(alg),
                "frac_measured": fmeas(achieved, stream_peak)}
        layer = {"bound": "hbm", "achieved": round(lay, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(lay / HBM_PEAK_GBS, 4), "frac_measured": fmeas(lay, stream_peak),
                 "alg_bytes_per_call": int(lay_b), "mean_active_experts": round(mean_active, 3),
                 "stage_ms": stages}
        at = curve_at(probes, lay_b)
        if at:
            layer["read_curve_gbs_at_layer_bytes"] = at
            layer["frac_of_curve_at_layer_bytes"] = round(lay / at, 4)
        if not fused:
            dn = sum(down_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
            layer["down_gbs"] = round(dn / (avg[2] * 1e-3) / 1e9, 1)
    log(f"[bench] roofline: {roof}")
    log(f"[bench] layer: {layer}")

    cpu = None
    if not args.no_cpu:
        t_cpu = {k: v[0] for k, v in inp.items()}
        cpu = cpu_baseline(wl, t_cpu, min_seconds=cpu_seconds)
        log(f"[bench] cpu oracle: {cpu}")
    del inp, ws, out
    torch.cuda.empty_cache()

    # arithmetic type of the expert dot products (weights x activations)
    dtype = {"bf16": "bf16", "f32": "f32", "q4_0": "q4_0xf16", "q8_0": "q8_0xf16", "fp8_e4m3": "fp8e4m3xbf16"}[wl.w_dtype]
    return {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "top_k": wl.k, "I": wl.I,
                   "n_shared": wl.S, "I_shared": wl.Is, "weights": wl.w_dtype, "activations": wl.x_dtype,
                   "router": wl.r_dtype, "path": path_name, "weight_copies": copies,
                   "timing": timing, "parallelism": "single-gpu"},
        "spread": spread,
        "isolated_call": isolated,
        "roofline": roof,
        "layer": layer,
        "cpu_baseline": cpu,
    }


# ------------------------------------------------------------------ main ----

# the workloads the metric names besides the headline: decode at batch one (the
# 256-expert Q4_0 layer), decode at batch 8 and 64 of the DeepSeek-shaped layer,
# and the 4096-token prefill
def measure_cache(args, m, wl, dev, n_layers=4, calls=48):
    """Costs of the host-resident expert cache on a decode layer shape.

    n_layers layers of routed experts live in pinned host memory.  Router
    biases fix each layer's experts: layer l engages experts (32 j + l) mod E,
    so that the next layer's experts are this layer's plus one -- the
    prefetch rule of the expert-cache page holds exactly.  Scenarios, each
    timed over `calls` calls that cycle through the layers (wall clock; every
    call waits for its routing anyway):
      resident   moe_forward with the layer's experts on the device (no cache);
      hit        every expert resident in the cache (slots >= all layers' experts);
      miss       the cache flushed before every call: every expert is read from
                 host memory by the kernels;
      no_prefetch  2 * top_k slots, no prefetch: each call's experts were
                 evicted by the two layers before it, so all miss;
      prefetch   2 * top_k slots, depth 1, shift 1: each call's experts were
                 predicted by the previous call and copied in meanwhile;
      prefetch_random  as prefetch, but the routing of each call is the
                 router's own (random) choice, so the prediction rarely holds.
    """
    import torch
    E, k = wl.E, wl.k
    shape = m.make_shape(wl.T, wl.H, wl.E, wl.I, k, wl.S, wl.Is, wl.x_dtype, wl.w_dtype, wl.r_dtype, 1)
    inp = synth.make_inputs_torch(wl, args.seed, device=dev, copies=n_layers)
    one = lambda key, l: inp[key][l] if isinstance(inp[key], list) else inp[key]  # noqa: E731
    host = []
    for l in range(n_layers):
        stacks = []
        for key in ("w_gate", "w_up", "w_down"):
            src = one(key, l).contiguous().view(torch.uint8).reshape(-1)
            h = torch.empty(src.numel(), dtype=torch.uint8, pin_memory=True)
            h.copy_(src)
            stacks.append(h)
        host.append(tuple(stacks))
    biases = []
    for l in range(n_layers):
        b = torch.zeros(E, dtype=torch.float32, device=dev)
        b[[(32 * j + l) % E for j in range(k)]] = 30.0
        biases.append(b)
    xs = [torch.randn(wl.T, wl.H, generator=torch.Generator(device=dev).manual_seed(100 + c), device=dev)
          .to(torch.float32 if wl.x_dtype == "f32" else torch.bfloat16) for c in range(calls)]
    ws = m.alloc_workspace(shape, dev)
    out = torch.empty_like(xs[0])
    copy = torch.cuda.Stream()

    def run(n_slots, depth, biased, flush=False, resident=False):
        region = torch.empty(m.moe_cache_region_bytes(shape, n_layers, n_slots), dtype=torch.uint8, device=dev)
        c = m.moe_cache_create(shape, host, region, n_slots, depth, 1, copy)
        try:
            def call(i):
                l = i % n_layers
                b = biases[l] if biased else None
                if resident:
                    m.moe_forward(shape, xs[i], one("router_w", l), b, one("w_gate", l), one("w_up", l),
                                  one("w_down", l), one("ws_gate", l), one("ws_up", l), one("ws_down", l), out, ws)
                    return
                if flush:
                    m.moe_cache_flush(c)
                m.moe_forward_cached(c, l, shape, xs[i], one("router_w", l), b, one("ws_gate", l), one("ws_up", l),
                                     one("ws_down", l), out, ws)
            # warm-up: three rounds over the layers, the host reading each round's routing (an
            # expert is copied in at its second miss), so the hit scenario starts all resident
            for r in range(3):
                for i in range(n_layers):
                    call(r * n_layers + i)
                torch.cuda.synchronize()
                copy.synchronize()
                m.moe_cache_stats(c)
            m.moe_cache_stats(c, reset=True)
            t0 = time.perf_counter()
            for i in range(calls):
                call(i)
            torch.cuda.synchronize()
            copy.synchronize()
            dt = time.perf_counter() - t0
            st = m.moe_cache_stats(c, reset=True)
        finally:
            torch.cuda.synchronize()
            m.moe_cache_destroy(c)
        r = {"us_per_call": round(dt / calls * 1e6, 2), "slots": n_slots, "prefetch_depth": depth}
        if not resident:
            r.update({kk: int(v) for kk, v in st.items()})
            r["h2d_gbs"] = round(st["bytes_copied"] / dt / 1e9, 2) if st["bytes_copied"] else 0.0
        return r

    res = {"resident": run(2 * k, 0, True, resident=True),
           "hit": run(n_layers * k, 0, True),
           "miss": run(2 * k, 0, True, flush=True),
           "no_prefetch": run(2 * k, 0, True),
           "prefetch": run(2 * k, 1, True),
           "prefetch_random": run(2 * k, 1, False)}
    expert_bytes = 2 * mat_bytes(wl.w_dtype, wl.I, wl.H) + mat_bytes(wl.w_dtype, wl.H, wl.I)
    return {"metric": "expert-cache layer call latency", "unit": "us/call", "higher_is_better": False,
            "n_gpus": 1, "data": "synthetic", "dtype": wl.w_dtype,
            "config": {"workload": wl.name, "layers": n_layers, "calls": calls, "expert_bytes": expert_bytes,
                       "T": wl.T, "E": E, "top_k": k, "routing": "router bias 30 on experts (32 j + layer) mod E"},
            "scenarios": res, "kernel_source_hash": kernel_source_hash()}


NESTED = ["qwen_a3b_decode_q4", "deepseek16b_decode_t8", "deepseek16b_decode_t64", "mixtral_prefill_t4096"]
HEADLINE = "mixtral_decode_t8"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the memory clocks settle within a few dozen steps)")
    ap.add_argument("--reps", type=int, default=5, help="repetitions of the timed loop for the spread")
    ap.add_argument("--workload", default=None, choices=sorted(synth.WORKLOADS),
                    help="time this workload only (default: the headline with the metric's other workloads nested)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = enough for ~10 GiB)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-probes", action="store_true", help="skip the bandwidth and MFMA probes")
    ap.add_argument("--graph", action="store_true", help="time hipGraph replays instead of eager launches")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "fused", "prefill"],
                    help="execution path (auto: the library's choice for the shape)")
    ap.add_argument("--cache", action="store_true",
                    help="instead: hit, miss and prefetch costs of the host-resident expert cache "
                         "(workload qwen_a3b_decode_q4 unless --workload is given)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              f"(the layer runs on a single MI355X; the design notes describe how it would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(2 ** 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB x5")
        return
    import mixture_experts_layer_12_amd as m
    if not os.path.exists(m.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    m.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.cache:
        rec = measure_cache(args, m, synth.WORKLOADS[args.workload or "qwen_a3b_decode_q4"], dev)
        print(json.dumps(rec), flush=True)
        return
    hip = HipEvents()
    single = args.workload is not None
    probes = None if (args.no_probes or single) else run_probes(m, dev, hip)
    rec = measure(args, m, synth.WORKLOADS[args.workload or HEADLINE], dev, hip, probes)
    if not single:
        rec["probes"] = probes
        rec["workloads"] = []
        for name in NESTED:
            if args.path != "auto":
                break
            rec["workloads"].append(measure(args, m, synth.WORKLOADS[name], dev, hip, probes, cpu_seconds=3.0))
    rec["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
