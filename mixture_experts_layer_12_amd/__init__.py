"""Python binding of the MoE layer C ABI (``include/moe.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``lib/libmoe.so``.  Functions carry the C names (``moe_workspace_size``,
``moe_dispatch_dims``, ``moe_route``, ``moe_forward``, ``moe_strerror``) and
accept torch tensors (their ``data_ptr()`` is passed) or raw integer device
addresses.  PyTorch only provides device memory and the current stream.

There is no fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe.so")

# enums of moe.h
MOE_F32, MOE_BF16, MOE_Q4_0, MOE_Q8_0, MOE_FP8_E4M3 = 0, 1, 2, 3, 4
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL, MOE_PATH_DECODE_FUSED = 0, 1, 2, 3
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
MOE_ERR_TOO_LARGE = -7
MOE_ERR_NOT_PINNED = -8
MOE_ERR_HOST_ALLOC = -9
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "q4_0": MOE_Q4_0, "q8_0": MOE_Q8_0, "fp8_e4m3": MOE_FP8_E4M3}
EXPORTED = ("moe_workspace_size", "moe_dispatch_dims", "moe_route", "moe_forward", "moe_forward_profiled",
            "moe_last_hip_error", "moe_strerror", "moe_resolve_path", "moe_sparse_workspace_size",
            "moe_forward_channel_sparse", "moe_forward_tables", "moe_route_workspace_size",
            "moe_probe_read", "moe_probe_mfma_bf16", "moe_forward_noalloc", "moe_cache_region_bytes",
            "moe_cache_create", "moe_cache_destroy", "moe_forward_cached", "moe_cache_stats", "moe_cache_flush")


class moe_shape_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "H", "E", "I", "top_k", "n_shared", "I_shared", "x_dtype", "w_dtype", "router_dtype", "path")]


class moe_route_out_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_ids", "topk_w", "counts", "offsets", "sorted_ids", "tile_expert", "inv", "active")]


class moe_forward_tables_t(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int32) for n in ("path", "tokens", "tile_m", "capacity", "n_tiles")] +
                [(n, ctypes.c_size_t) for n in ("topk_ids", "topk_w", "counts", "offsets", "sorted_ids",
                                                "tile_expert", "inv", "active", "status")] +
                [(n, ctypes.c_int32) for n in ("route_in_gateup", "shared_in_router")])


class moe_host_experts_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down")]


class moe_cache_stats_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "lookups", "hits", "misses", "prefetches", "prefetch_hits", "bytes_copied")]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {moe_strerror(code)} ({code})"
        if code == MOE_ERR_HIP:
            msg += f"; {hip_error_name(moe_last_hip_error())}"
        super().__init__(msg)


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises FileNotFoundError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.moe_workspace_size.argtypes = [P(moe_shape_t), P(sz)]
    lib.moe_workspace_size.restype = ctypes.c_int
    lib.moe_dispatch_dims.argtypes = [P(moe_shape_t), P(i32), P(i32), P(i32)]
    lib.moe_dispatch_dims.restype = ctypes.c_int
    lib.moe_route.argtypes = [P(moe_shape_t), vp, vp, vp, P(moe_route_out_t), vp, sz, vp]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_forward.argtypes = [P(moe_shape_t), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_profiled.argtypes = [P(moe_shape_t), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                         P(vp), ctypes.c_int]
    lib.moe_forward_profiled.restype = ctypes.c_int
    lib.moe_last_hip_error.argtypes = []
    lib.moe_last_hip_error.restype = ctypes.c_int
    lib.moe_sparse_workspace_size.argtypes = [P(moe_shape_t), i32, P(sz)]
    lib.moe_sparse_workspace_size.restype = ctypes.c_int
    lib.moe_forward_channel_sparse.argtypes = [P(moe_shape_t), i32] + [vp] * 12 + [sz, vp]
    lib.moe_forward_channel_sparse.restype = ctypes.c_int
    lib.moe_forward_tables.argtypes = [P(moe_shape_t), P(moe_forward_tables_t)]
    lib.moe_forward_tables.restype = ctypes.c_int
    lib.moe_route_workspace_size.argtypes = [P(moe_shape_t), P(sz)]
    lib.moe_route_workspace_size.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [P(moe_shape_t), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_probe_read.argtypes = [vp, sz, vp, vp]
    lib.moe_probe_read.restype = ctypes.c_int
    lib.moe_probe_mfma_bf16.argtypes = [i32, vp, P(ctypes.c_double), vp]
    lib.moe_probe_mfma_bf16.restype = ctypes.c_int
    lib.moe_cache_region_bytes.argtypes = [P(moe_shape_t), i32, i32, P(sz)]
    lib.moe_cache_region_bytes.restype = ctypes.c_int
    lib.moe_cache_create.argtypes = [P(moe_shape_t), i32, P(moe_host_experts_t), vp, sz, i32, i32, i32, vp,
                                     P(vp)]
    lib.moe_cache_create.restype = ctypes.c_int
    lib.moe_cache_destroy.argtypes = [vp]
    lib.moe_cache_destroy.restype = ctypes.c_int
    lib.moe_forward_cached.argtypes = [vp, i32, P(moe_shape_t), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward_cached.restype = ctypes.c_int
    lib.moe_cache_stats.argtypes = [vp, P(moe_cache_stats_t), i32]
    lib.moe_cache_stats.restype = ctypes.c_int
    lib.moe_cache_flush.argtypes = [vp]
    lib.moe_cache_flush.restype = ctypes.c_int
    lib.moe_resolve_path.argtypes = [P(moe_shape_t)]
    lib.moe_resolve_path.restype = ctypes.c_int
    lib.moe_strerror.argtypes = [ctypes.c_int]
    lib.moe_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_shape(T, H, E, I, top_k, n_shared=0, I_shared=0, x_dtype="bf16", w_dtype="bf16",
               router_dtype="bf16", path=MOE_PATH_AUTO) -> moe_shape_t:
    conv = lambda d: DTYPES[d] if isinstance(d, str) else int(d)
    return moe_shape_t(int(T), int(H), int(E), int(I), int(top_k), int(n_shared), int(I_shared),
                       conv(x_dtype), conv(w_dtype), conv(router_dtype), int(path))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def moe_strerror(code: int) -> str:
    return load_library().moe_strerror(int(code)).decode()


def moe_last_hip_error() -> int:
    return int(load_library().moe_last_hip_error())


def hip_error_name(err: int) -> str:
    """hipGetErrorName of a hipError_t value (from the HIP runtime)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipGetErrorName.restype = ctypes.c_char_p
        hip.hipGetErrorName.argtypes = [ctypes.c_int]
        return f"hipError {err} ({hip.hipGetErrorName(err).decode()})"
    except OSError:
        return f"hipError {err}"


def moe_sparse_workspace_size(shape: moe_shape_t, budget: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().moe_sparse_workspace_size(ctypes.byref(shape), int(budget), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_sparse_workspace_size")
    return n.value


def moe_forward_channel_sparse(shape: moe_shape_t, budget: int, channel_scores, x, router_w, router_b, w_gate, w_up,
                               w_down_t, ws_gate, ws_up, ws_down, out, workspace, ws_bytes=None, stream=None,
                               check=True) -> int:
    nb = _nbytes(workspace) if ws_bytes is None else ws_bytes
    rc = load_library().moe_forward_channel_sparse(
        ctypes.byref(shape), int(budget), _ptr(channel_scores), _ptr(x), _ptr(router_w), _ptr(router_b),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down_t), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(out),
        _ptr(workspace), nb, _stream(stream))
    if check and rc:
        raise MoeError(rc, "moe_forward_channel_sparse")
    return rc


def moe_resolve_path(shape: moe_shape_t) -> int:
    """MOE_PATH_DECODE / _PREFILL / _DECODE_FUSED that moe_forward takes for ``shape``."""
    rc = load_library().moe_resolve_path(ctypes.byref(shape))
    if rc < 0:
        raise MoeError(rc, "moe_resolve_path")
    return rc


def moe_workspace_size(shape: moe_shape_t) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_workspace_size")
    return n.value


def moe_probe_read(buf, nbytes: int, sink, stream=None) -> None:
    """Measurement probe (include/moe_probe.h): read ``nbytes`` of ``buf`` once."""
    rc = load_library().moe_probe_read(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_probe_read")


def moe_probe_mfma_bf16(iters: int, sink, stream=None) -> float:
    """Measurement probe: back-to-back bf16 MFMAs on every compute unit; returns the launch's flops."""
    fl = ctypes.c_double(0.0)
    rc = load_library().moe_probe_mfma_bf16(int(iters), _ptr(sink), ctypes.byref(fl), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_probe_mfma_bf16")
    return fl.value


def moe_route_workspace_size(shape: moe_shape_t) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().moe_route_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_route_workspace_size")
    return n.value


def moe_forward_tables(shape: moe_shape_t) -> dict:
    """Where moe_forward leaves the routing of its last pass in the workspace:
    path, tokens, tile_m, capacity, n_tiles and the byte offsets of the arrays."""
    t = moe_forward_tables_t()
    rc = load_library().moe_forward_tables(ctypes.byref(shape), ctypes.byref(t))
    if rc:
        raise MoeError(rc, "moe_forward_tables")
    return {n: getattr(t, n) for n, _ in moe_forward_tables_t._fields_}


def fused_status_ok(shape: moe_shape_t, workspace) -> bool:
    """After a completed call whose shape has status words (the single-launch
    decode, or a decode pass whose selection runs inside the logits launch):
    True unless a wait gave up (the two status words of moe_forward_tables_t
    are equal).  Reads 16 bytes of the workspace back to the host; the caller
    synchronises first."""
    import torch
    o = moe_forward_tables(shape)["status"]
    if o == 0:
        raise ValueError("no status words for this shape and path")
    w = workspace[o:o + 16].view(torch.int64).cpu()
    return int(w[0]) != int(w[1])


def moe_dispatch_dims(shape: moe_shape_t):
    """(tile_m, capacity, n_tiles) of the expert-sorted order."""
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().moe_dispatch_dims(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    if rc:
        raise MoeError(rc, "moe_dispatch_dims")
    return a.value, b.value, c.value


def moe_route(shape: moe_shape_t, x, router_w, router_b, out: dict, workspace, ws_bytes=None, stream=None,
              check=True) -> int:
    """``out`` maps moe_route_out_t field names to int32/float32 device tensors (or None)."""
    ro = moe_route_out_t(*[_ptr(out.get(n)) for n, _ in moe_route_out_t._fields_])
    nb = _nbytes(workspace) if ws_bytes is None else ws_bytes
    rc = load_library().moe_route(ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(router_b), ctypes.byref(ro),
                                  _ptr(workspace), nb, _stream(stream))
    if check and rc:
        raise MoeError(rc, "moe_route")
    return rc


def moe_forward(shape: moe_shape_t, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                out, workspace, ws_bytes=None, stream=None, check=True) -> int:
    nb = _nbytes(workspace) if ws_bytes is None else ws_bytes
    rc = load_library().moe_forward(ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(router_b),
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                                    _ptr(ws_down), _ptr(out), _ptr(workspace), nb, _stream(stream))
    if check and rc:
        raise MoeError(rc, "moe_forward")
    return rc


def moe_forward_noalloc(shape: moe_shape_t, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                        out, stream=None, check=True) -> int:
    """moe_forward with the library's static device scratch as its workspace (allocates nothing)."""
    rc = load_library().moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(router_b),
                                            _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                                            _ptr(ws_down), _ptr(out), _stream(stream))
    if check and rc:
        raise MoeError(rc, "moe_forward_noalloc")
    return rc


def moe_forward_profiled(shape: moe_shape_t, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up,
                         ws_down, out, workspace, events, ws_bytes=None, stream=None, check=True) -> int:
    """``events``: sequence of raw hipEvent_t handles (ints) recorded at stage boundaries."""
    nb = _nbytes(workspace) if ws_bytes is None else ws_bytes
    arr = (ctypes.c_void_p * len(events))(*events)
    rc = load_library().moe_forward_profiled(ctypes.byref(shape), _ptr(x), _ptr(router_w), _ptr(router_b),
                                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                                             _ptr(ws_down), _ptr(out), _ptr(workspace), nb, _stream(stream),
                                             arr, len(events))
    if check and rc:
        raise MoeError(rc, "moe_forward_profiled")
    return rc


def moe_cache_region_bytes(shape: moe_shape_t, n_layers: int, n_slots: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().moe_cache_region_bytes(ctypes.byref(shape), n_layers, n_slots, ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_cache_region_bytes")
    return n.value


def moe_cache_create(shape: moe_shape_t, layers, region, n_slots: int, prefetch_depth: int, prefetch_shift: int,
                     copy_stream, region_bytes=None, check=True):
    """``layers``: sequence of (w_gate, w_up, w_down) pinned host buffers per layer.  Returns the
    handle (an int), or the error code when ``check`` is false and the call fails."""
    arr = (moe_host_experts_t * len(layers))(*[moe_host_experts_t(_ptr(g), _ptr(u), _ptr(d)) for g, u, d in layers])
    h = ctypes.c_void_p(None)
    nb = _nbytes(region) if region_bytes is None else region_bytes
    rc = load_library().moe_cache_create(ctypes.byref(shape), len(layers), arr, _ptr(region), nb, n_slots,
                                         prefetch_depth, prefetch_shift, _stream(copy_stream), ctypes.byref(h))
    if rc:
        if check:
            raise MoeError(rc, "moe_cache_create")
        return rc
    return h.value


def moe_cache_destroy(cache) -> None:
    rc = load_library().moe_cache_destroy(cache)
    if rc:
        raise MoeError(rc, "moe_cache_destroy")


def moe_forward_cached(cache, layer: int, shape: moe_shape_t, x, router_w, router_b, ws_gate, ws_up, ws_down, out,
                       workspace, ws_bytes=None, stream=None, check=True) -> int:
    nb = _nbytes(workspace) if ws_bytes is None else ws_bytes
    rc = load_library().moe_forward_cached(cache, layer, ctypes.byref(shape), _ptr(x), _ptr(router_w),
                                           _ptr(router_b), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(out),
                                           _ptr(workspace), nb, _stream(stream))
    if check and rc:
        raise MoeError(rc, "moe_forward_cached")
    return rc


def moe_cache_stats(cache, reset: bool = False) -> dict:
    st = moe_cache_stats_t()
    rc = load_library().moe_cache_stats(cache, ctypes.byref(st), 1 if reset else 0)
    if rc:
        raise MoeError(rc, "moe_cache_stats")
    return {n: getattr(st, n) for n, _ in moe_cache_stats_t._fields_}


def moe_cache_flush(cache) -> None:
    rc = load_library().moe_cache_flush(cache)
    if rc:
        raise MoeError(rc, "moe_cache_flush")


def alloc_sparse_workspace(shape: moe_shape_t, budget: int, device="cuda"):
    """A workspace of moe_sparse_workspace_size(shape, budget) bytes (contents irrelevant)."""
    import torch
    return torch.empty(max(moe_sparse_workspace_size(shape, budget), 256), dtype=torch.uint8, device=device)


def alloc_workspace(shape: moe_shape_t, device="cuda"):
    """A workspace of moe_workspace_size(shape) bytes (torch uint8 tensor; contents irrelevant)."""
    import torch
    return torch.empty(max(moe_workspace_size(shape), 256), dtype=torch.uint8, device=device)
