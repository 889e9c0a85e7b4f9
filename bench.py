#!/usr/bin/env python3
"""Throughput of the fused MoE layer forward on one MI355X.

One step = one whole layer call (router + dispatch, expert gate/up, expert
down + weighted combine) through the C ABI on one batch of synthetic inputs
already resident in HBM.  The default workload is the Mixtral-8x7B-shaped
decode layer (T=8 tokens, hidden 4096, 8 experts, top-2, SwiGLU intermediate
14336, bf16 weights).  Weight sets are rotated between steps so that every
step streams its weights from HBM rather than from the 256 MB Infinity Cache.

Prints ONE JSON line on stdout.  Besides the throughput it carries
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                divided by its average launch duration, measured with HIP
                events recorded on the launch stream around that kernel;
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample.

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

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0)
            if rc:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            evs.append(e.value)
        return evs

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


def gateup_alg_bytes(wl, n_active, T):
    """Algorithmic bytes of one decode gate/up launch: the engaged experts' gate
    and up rows, the activations read and the intermediate rows written."""
    return (n_active * 2 * mat_bytes(wl.w_dtype, wl.I, wl.H) + wl.S * 2 * mat_bytes(wl.w_dtype, wl.Is, wl.H)
            + T * wl.H * act_bytes(wl.x_dtype) + (T * wl.k * wl.I + wl.S * T * wl.Is) * h_elem_bytes(wl))


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
    h = hashlib.sha256()
    for f in ("common.hpp", "decode_items.hpp", "router_items.hpp", "decode.hip", "decode_fused.hip", "prefill.hip",
              "router.hip"):
        with open(os.path.join(ROOT, "mixture_experts_layer_12_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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

def cpu_baseline(wl, t, tokens_max=16, min_seconds=5.0):
    """The fp64 oracle on a bounded sample of the same workload: the first
    min(T, tokens_max) tokens of weight copy 0, decoding from the stored bits
    only the experts those tokens reach.  Repeated until min_seconds."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_info

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
    return {"value": reps * n_tok / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tok} of {wl.T} tokens of one layer call (weight copy 0), x{reps} repetitions, "
                      f"fp64 numpy oracle including decoding the stored weights of the experts those tokens reach; "
                      f"{el:.1f} s",
            "host_cpus": os.cpu_count()}


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
    print(json.dumps(rec), flush=True)


# ------------------------------------------------------------------ main ----

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_decode_t8", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = enough for ~10 GiB)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action="store_true", help="time hipGraph replays instead of eager launches")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "fused", "prefill"],
                    help="execution path (auto: the library's choice for the shape)")
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

    wl = synth.WORKLOADS[args.workload]
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

    # eager warm-up (also performs the library's one-time set-up before any capture)
    torch.cuda.synchronize()
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    eager_elapsed = timed(step, args.steps, args.warmup)
    eager_value = wl.T * args.steps / eager_elapsed
    graph_value = None

    if not args.graph:
        elapsed = eager_elapsed
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
        replay = lambda i: graphs[i % copies].replay()
        for i in range(args.warmup):
            replay(i)
        elapsed = timed(replay, args.steps, args.warmup)
        graph_value = wl.T * args.steps / elapsed
        timing = "hipGraph replay, one graph per weight copy"
    log(f"[bench] warmup {args.warmup}; timed {args.steps} steps ({timing})")
    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, {value:.1f} tokens/s (eager {eager_value:.1f} tokens/s)")

    # stage timing with HIP events recorded on the launch stream
    prefill = path_name == "prefill"
    fused = path_name == "decode_fused"
    n_ev = 5 if prefill else (2 if fused else 4)
    hip = HipEvents()
    evs = [hip.create(n_ev) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    stage = [[hip.elapsed_ms(e[j], e[j + 1]) for j in range(n_ev - 1)] for e in evs]
    for e in evs:
        hip.destroy(e)
    avg = [sum(s[j] for s in stage) / len(stage) for j in range(n_ev - 1)]
    names = (["router", "prefill_gateup", "prefill_down", "cast"] if prefill
             else (["decode_fused"] if fused else ["router", "decode_gateup", "decode_down"]))
    log("[bench] stage averages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in zip(names, avg)))

    # engaged experts per weight copy (from the run's own routing)
    n_active = []
    for c in range(copies):
        r_out = dict(topk_ids=torch.empty(wl.T * wl.k, dtype=torch.int32, device=dev),
                     topk_w=torch.empty(wl.T * wl.k, dtype=torch.float32, device=dev),
                     active=torch.empty(wl.E + 1, dtype=torch.int32, device=dev))
        m.moe_route(shape, inp["x"][c], inp["router_w"][c], inp["router_b"][c], r_out, ws, stream=sh)
        torch.cuda.synchronize()
        n_active.append(int(r_out["active"][0].item()))
    steps_copies = [(args.warmup + i) % copies for i in range(args.steps)]
    mean_active = sum(n_active[c] for c in steps_copies) / args.steps

    if prefill:
        kname = "prefill_gateup"
        fl = gateup_flops(wl)
        achieved = fl / (avg[1] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(wl.name, kname),
                "kernel": kname, "launch_ms": round(avg[1], 5), "alg_flops_per_launch": fl,
                "layer_tflops": round(layer_flops(wl) / (ms_per_step * 1e-3) / 1e12, 2)}
    elif fused:
        # one launch runs the whole layer: its algorithmic bytes over its duration
        kname = "decode_fused"
        lay = sum(layer_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
        achieved = lay / (avg[0] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name, kname),
                "kernel": kname, "launch_ms": round(avg[0], 5), "alg_bytes_per_launch": int(lay),
                "mean_active_experts": round(mean_active, 3),
                "layer_gbs": round(lay / (ms_per_step * 1e-3) / 1e9, 1)}
    else:
        kname = "decode_gateup"
        alg = sum(gateup_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
        achieved = alg / (avg[1] * 1e-3) / 1e9
        lay = sum(layer_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
        dn = sum(down_alg_bytes(wl, n_active[c], wl.T) for c in steps_copies) / args.steps
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name, kname),
                "kernel": kname, "launch_ms": round(avg[1], 5), "alg_bytes_per_launch": int(alg),
                "mean_active_experts": round(mean_active, 3),
                "down_kernel_gbs": round(dn / (avg[2] * 1e-3) / 1e9, 1),
                "layer_gbs": round(lay / (ms_per_step * 1e-3) / 1e9, 1)}
    log(f"[bench] roofline: {roof}")

    cpu = None
    if not args.no_cpu:
        t_cpu = {k: v[0] for k, v in inp.items()}
        cpu = cpu_baseline(wl, t_cpu)
        log(f"[bench] cpu oracle: {cpu}")

    # arithmetic type of the expert dot products (weights x activations)
    dtype = {"bf16": "bf16", "f32": "f32", "q4_0": "q4_0xf16", "q8_0": "q8_0xf16", "fp8_e4m3": "fp8e4m3xbf16"}[wl.w_dtype]
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "top_k": wl.k, "I": wl.I,
                   "n_shared": wl.S, "I_shared": wl.Is, "weights": wl.w_dtype, "activations": wl.x_dtype,
                   "router": wl.r_dtype, "path": path_name, "weight_copies": copies,
                   "timing": timing, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
