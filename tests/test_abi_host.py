"""Host-side checks of the C ABI (no GPU needed, no kernel launched): the
library loads, exports every function include/moe.h declares, and rejects bad
arguments with the documented codes before touching the GPU."""
import ctypes
import os
import re

import pytest

from tests import helpers as H


@pytest.fixture(scope="module")
def m():
    return H.lib()


def _declared(root):
    names = set()
    for h in sorted(os.listdir(os.path.join(root, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(root, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(m, root):
    names = _declared(root)
    assert set(names) == set(m.EXPORTED)
    lib = m.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding(m, root):
    text = open(os.path.join(root, "include", "moe.h")).read()
    for name, val in [("MOE_ERR_WORKSPACE", -5), ("MOE_ERR_HIP", -6), ("MOE_PATH_PREFILL", 2), ("MOE_Q4_0", 2)]:
        assert re.search(rf"{name}\s*=\s*{val}", text), name


def test_strerror(m):
    assert m.moe_strerror(0) == "ok"
    assert "workspace" in m.moe_strerror(m.MOE_ERR_WORKSPACE)
    assert m.moe_strerror(12345) == "unknown error code"


@pytest.mark.parametrize("kw, code", [
    (dict(H=100), "MOE_ERR_SHAPE"),          # H % 32 != 0
    (dict(I=0), "MOE_ERR_SHAPE"),
    (dict(E=0), "MOE_ERR_SHAPE"),
    (dict(E=257, top_k=2), "MOE_ERR_SHAPE"),
    (dict(top_k=9), "MOE_ERR_SHAPE"),        # k > E
    (dict(top_k=0), "MOE_ERR_SHAPE"),
    (dict(T=-1), "MOE_ERR_SHAPE"),
    (dict(n_shared=1, I_shared=33), "MOE_ERR_SHAPE"),
    (dict(x_dtype=2), "MOE_ERR_DTYPE"),      # Q4_0 activations
    (dict(router_dtype=7), "MOE_ERR_DTYPE"),
    (dict(w_dtype=5), "MOE_ERR_DTYPE"),
    (dict(w_dtype=2, path=2), "MOE_ERR_DTYPE"),  # prefill needs bf16 experts
    (dict(path=4), "MOE_ERR_SHAPE"),
    (dict(w_dtype=3, path=2), "MOE_ERR_DTYPE"),   # the 8-bit weight types run the decode path only
    (dict(w_dtype=4, path=3), "MOE_ERR_DTYPE"),
    (dict(path=3, router_dtype=0), "MOE_ERR_DTYPE"),   # single-launch decode: router dtype == x dtype
    (dict(path=3, E=32, top_k=17), "MOE_ERR_SHAPE"),    # single-launch decode: top_k <= 16
])
def test_shape_validation(m, kw, code):
    base = dict(T=8, H=256, E=8, I=128, top_k=2, n_shared=0, I_shared=0, x_dtype=1, w_dtype=1,
                router_dtype=1, path=0)
    base.update(kw)
    s = m.moe_shape_t(*[base[n] for n, _ in m.moe_shape_t._fields_])
    n = ctypes.c_size_t(0)
    assert m.load_library().moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == getattr(m, code)


@pytest.mark.parametrize("kw, budget, code", [
    (dict(), 0, "MOE_ERR_SHAPE"),
    (dict(), 129, "MOE_ERR_SHAPE"),                       # budget > I
    (dict(w_dtype=2), 8, "MOE_ERR_DTYPE"),                # dense f32 / bf16 experts only
    (dict(I=16416), 8, "MOE_ERR_SHAPE"),                  # I above the selection's LDS limit
])
def test_sparse_validation(m, kw, budget, code):
    base = dict(T=4, H=256, E=8, I=128, top_k=2, n_shared=0, I_shared=0, x_dtype=1, w_dtype=1,
                router_dtype=1, path=0)
    base.update(kw)
    s = m.moe_shape_t(*[base[n] for n, _ in m.moe_shape_t._fields_])
    n = ctypes.c_size_t(0)
    assert m.load_library().moe_sparse_workspace_size(ctypes.byref(s), budget, ctypes.byref(n)) == getattr(m, code)


def test_sparse_workspace_grows_with_budget(m):
    s = m.make_shape(1, 4096, 8, 14336, 2)
    assert m.moe_sparse_workspace_size(s, 2552) > m.moe_sparse_workspace_size(s, 256) > 0


def test_resolve_path(m):
    P = m
    assert m.moe_resolve_path(m.make_shape(8, 4096, 8, 14336, 2)) == P.MOE_PATH_DECODE
    assert m.moe_resolve_path(m.make_shape(8, 4096, 8, 14336, 2, path=3)) == P.MOE_PATH_DECODE_FUSED
    assert m.moe_resolve_path(m.make_shape(4096, 4096, 8, 14336, 2)) == P.MOE_PATH_PREFILL
    # router dtype differs from the activations: multi-launch decode
    assert m.moe_resolve_path(m.make_shape(8, 256, 8, 128, 2, x_dtype="f32", router_dtype="bf16")) == P.MOE_PATH_DECODE
    assert m.moe_resolve_path(m.make_shape(4, 64, 64, 32, 20)) == P.MOE_PATH_DECODE          # top_k > 16
    assert m.moe_resolve_path(m.make_shape(100, 64, 8, 32, 2, x_dtype="f32", w_dtype="f32",
                                           router_dtype="f32", path=3)) == P.MOE_PATH_DECODE_FUSED
    assert m.moe_resolve_path(m.make_shape(8, 256, 8, 128, 2, path=1)) == P.MOE_PATH_DECODE
    with pytest.raises(m.MoeError):
        m.moe_resolve_path(m.make_shape(8, 100, 8, 128, 2))


def test_single_launch_decode_workspace(m):
    """The single-launch decode adds completion flags to the decode workspace;
    the multi-launch decode of the same shape cuts its down projection into 2
    k ranges instead and holds one more plane of partial rows, and the flags
    and status pair of a selection inside the logits launch (one aligned
    block each)."""
    fused = m.moe_workspace_size(m.make_shape(8, 4096, 8, 14336, 2, path=m.MOE_PATH_DECODE_FUSED))
    multi = m.moe_workspace_size(m.make_shape(8, 4096, 8, 14336, 2, path=m.MOE_PATH_DECODE))
    plane = 16 * 4096 * 4 + 2 * 256    # T*k = 16 partial rows of H = 4096 floats; selection flags, status

    # work list: 4 logits planes, 1 selection, 8 x 896 gate/up tiles, 8 x 128 down row groups (32 outputs
    # each), 32 combine blocks
    n_items = 4 + 1 + 8 * 896 + 8 * 128 + 32
    assert fused - (multi - plane) >= n_items * 8
    assert fused - (multi - plane) < n_items * 8 + 4096


def test_workspace_size_and_dims(m):
    s = m.make_shape(4096, 4096, 8, 14336, 2)
    tile_m, cap, n_tiles = m.moe_dispatch_dims(s)
    assert tile_m == 128 and cap == (4096 * 2 + 8 * 127 + 127) // 128 * 128 and n_tiles * tile_m == cap
    big = m.moe_workspace_size(s)
    # prefill needs the bf16 activations and the down GEMM's fp32 partial rows: two k ranges
    # (planes) of at least the T*k routed rows
    assert big >= cap * 14336 * 2 + 2 * (4096 * 2) * 4096 * 4
    small = m.moe_workspace_size(m.make_shape(8, 4096, 8, 14336, 2))
    assert 0 < small < big


def test_argument_errors_before_launch(m):
    """Error paths return before any HIP call (safe without a GPU)."""
    lib = m.load_library()
    s = m.make_shape(8, 256, 8, 128, 2)
    fake = 1 << 20                      # never dereferenced: validation fails first
    nb = m.moe_workspace_size(s)
    ro = m.moe_route_out_t(fake, fake, None, None, None, None, None, None)
    # missing weights
    rc = lib.moe_forward(ctypes.byref(s), fake, fake, None, None, fake, fake, None, None, None, fake, fake, nb, None)
    assert rc == m.MOE_ERR_NULL
    # shared weights given with n_shared == 0
    rc = lib.moe_forward(ctypes.byref(s), fake, fake, None, fake, fake, fake, fake, fake, fake, fake, fake, nb, None)
    assert rc == m.MOE_ERR_NULL
    # misaligned pointer
    rc = lib.moe_forward(ctypes.byref(s), fake + 4, fake, None, fake, fake, fake, None, None, None, fake, fake, nb, None)
    assert rc == m.MOE_ERR_ALIGN
    # workspace too small
    rc = lib.moe_forward(ctypes.byref(s), fake, fake, None, fake, fake, fake, None, None, None, fake, fake, nb - 1, None)
    assert rc == m.MOE_ERR_WORKSPACE
    rc = lib.moe_route(ctypes.byref(s), fake, fake, None, ctypes.byref(ro), fake, 16, None)
    assert rc == m.MOE_ERR_WORKSPACE
    ro2 = m.moe_route_out_t(None, fake, None, None, None, None, None, None)
    assert lib.moe_route(ctypes.byref(s), fake, fake, None, ctypes.byref(ro2), fake, nb, None) == m.MOE_ERR_NULL
    # T == 0 is a no-op that touches nothing
    s0 = m.make_shape(0, 256, 8, 128, 2)
    assert lib.moe_forward(ctypes.byref(s0), None, None, None, None, None, None, None, None, None, None, None,
                           0, None) == m.MOE_OK


def _shape(m, **kw):
    base = dict(T=8, H=256, E=8, I=128, top_k=2, n_shared=0, I_shared=0, x_dtype=1, w_dtype=1,
                router_dtype=1, path=0)
    base.update(kw)
    return m.moe_shape_t(*[base[n] for n, _ in m.moe_shape_t._fields_])


@pytest.mark.parametrize("kw, path, tokens, tile_m", [
    (dict(T=8), 1, 8, 1),                    # one decode pass, no padding
    (dict(T=70, w_dtype=2), 1, 6, 1),        # decode passes of 64: the last pass holds 6 tokens
    (dict(T=64), 1, 64, 1),
    (dict(T=300), 2, 300, 256),              # prefill, segments padded to 256 rows
    (dict(T=8, path=3), 3, 8, 1),            # single-launch decode
])
def test_forward_tables_layout(m, kw, path, tokens, tile_m):
    s = _shape(m, **kw)
    t = m.moe_forward_tables(s)
    assert (t["path"], t["tokens"], t["tile_m"]) == (path, tokens, tile_m)
    k, E = s.top_k, s.E
    n = tokens * k
    if tile_m == 1:
        assert t["capacity"] == n and t["n_tiles"] == 0 and t["tile_expert"] == 0
    else:
        assert t["capacity"] == -(-(n + E * (tile_m - 1)) // tile_m) * tile_m
        assert t["n_tiles"] == t["capacity"] // tile_m
    ws = m.moe_workspace_size(s)
    spans = [(t["topk_ids"], 4 * n), (t["topk_w"], 4 * n), (t["counts"], 4 * E), (t["offsets"], 4 * (E + 1)),
             (t["sorted_ids"], 4 * t["capacity"]), (t["inv"], 4 * n), (t["active"], 4 * (E + 1))]
    if t["n_tiles"]:
        spans.append((t["tile_expert"], 4 * t["n_tiles"]))
    spans.sort()
    for (o, b), (o2, _) in zip(spans, spans[1:]):
        assert o % 16 == 0 and o + b <= o2              # aligned, disjoint
    assert spans[-1][0] + spans[-1][1] <= ws


def test_route_workspace_is_at_most_the_forward_workspace(m):
    for kw in (dict(T=8), dict(T=4096, I=14336, H=4096), dict(T=1, E=256, top_k=8, w_dtype=2)):
        s = _shape(m, **kw)
        assert 0 < m.moe_route_workspace_size(s) <= m.moe_workspace_size(s)
    # moe_route rejects a workspace below its own size before touching the GPU
    s = _shape(m, T=8)
    need = m.moe_route_workspace_size(s)
    buf = (ctypes.c_int32 * 16)()
    out = m.moe_route_out_t(ctypes.addressof(buf), ctypes.addressof(buf), None, None, None, None, None, None)
    p = ctypes.addressof(buf)
    assert m.load_library().moe_route(ctypes.byref(s), p, p, None, ctypes.byref(out), p, need - 1,
                                      None) == m.MOE_ERR_WORKSPACE


def _stack_bytes(w_dtype, n, N, K):
    """Bytes of a stack of n matrices [N, K] in the layouts moe.h states."""
    up = lambda v: -(-v // 256) * 256  # noqa: E731
    if w_dtype == 0:
        return n * N * K * 4
    if w_dtype == 1:
        return n * N * K * 2
    if w_dtype == 2:
        return up(n * N * K // 2) + n * N * (K // 32) * 2
    if w_dtype == 3:
        return up(n * N * K) + n * N * (K // 32) * 2
    return up(n * N * K) + n * N * 4


@pytest.mark.parametrize("w_dtype", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n_layers, n_slots", [(1, 1), (3, 5), (48, 64)])
def test_cache_region_bytes(m, w_dtype, n_layers, n_slots):
    up = lambda v: -(-v // 256) * 256  # noqa: E731
    s = _shape(m, T=1, H=256, E=16, I=96, top_k=4, w_dtype=w_dtype)
    want = up(4 * n_layers * s.E)                   # the slot map
    for N, K in ((s.I, s.H), (s.I, s.H), (s.H, s.I)):
        want += up(_stack_bytes(w_dtype, n_slots, N, K))
    assert m.moe_cache_region_bytes(s, n_layers, n_slots) == want


def test_cache_argument_errors_on_the_host(m):
    lib = m.load_library()
    s = _shape(m, T=1)
    n = ctypes.c_size_t(0)
    assert lib.moe_cache_region_bytes(ctypes.byref(s), 1, 0, ctypes.byref(n)) == m.MOE_ERR_SHAPE
    assert lib.moe_cache_region_bytes(ctypes.byref(s), 0, 4, ctypes.byref(n)) == m.MOE_ERR_SHAPE
    assert lib.moe_cache_region_bytes(ctypes.byref(_shape(m, H=100)), 1, 4, ctypes.byref(n)) == m.MOE_ERR_SHAPE
    h = ctypes.c_void_p(None)
    layer = m.moe_host_experts_t(None, None, None)
    big = m.moe_cache_region_bytes(s, 1, 4)
    buf = (ctypes.c_uint8 * (big + 256))()
    region = (ctypes.addressof(buf) + 255) // 256 * 256
    # no layers / no region / no handle
    assert lib.moe_cache_create(ctypes.byref(s), 1, None, region, 512, 4, 0, 0, region, ctypes.byref(h)) == \
        m.MOE_ERR_NULL
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), None, 512, 4, 0, 0, region,
                                ctypes.byref(h)) == m.MOE_ERR_NULL
    # a region below moe_cache_region_bytes, a prefetch depth of n_layers, no copy stream, NULL stacks
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), region, 512, 4, 0, 0, region,
                                ctypes.byref(h)) == m.MOE_ERR_WORKSPACE
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), region + 16, big, 4, 0, 0, region,
                                ctypes.byref(h)) == m.MOE_ERR_ALIGN
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), region, big, 4, 1, 0, region,
                                ctypes.byref(h)) == m.MOE_ERR_SHAPE
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), region, big, 4, 0, 0, None,
                                ctypes.byref(h)) == m.MOE_ERR_NULL
    assert lib.moe_cache_create(ctypes.byref(s), 1, ctypes.byref(layer), region, big, 4, 0, 0, region,
                                ctypes.byref(h)) == m.MOE_ERR_NULL
    assert h.value is None
    st = m.moe_cache_stats_t()
    assert lib.moe_cache_stats(None, ctypes.byref(st), 0) == m.MOE_ERR_NULL
    assert lib.moe_cache_flush(None) == m.MOE_ERR_NULL
    assert lib.moe_cache_destroy(None) == m.MOE_ERR_NULL
    assert lib.moe_forward_cached(None, 0, ctypes.byref(s), *([None] * 8), 0, None) == m.MOE_ERR_NULL


@pytest.mark.parametrize("kw, route_in_gateup, shared_in_router", [
    (dict(T=1, H=2048, E=256, I=512, top_k=8, n_shared=1, I_shared=512, w_dtype=2), 1, 1),  # Qwen-A3B-shaped
    (dict(T=8, H=4096, E=8, I=14336, top_k=2), 1, 0),          # tiny selection on a large grid
    (dict(T=8, H=4096, E=8, I=14336, top_k=2, w_dtype=4), 0, 0),   # ... but not with fp8 weights
    # too many groups for the routing in the gate/up prologue: the shared gate/up and the selection
    # in the logits launch
    (dict(T=8, H=2048, E=64, I=1408, top_k=6, n_shared=2, I_shared=1408), 0, 1),
    (dict(T=40, E=16, top_k=2), 0, 0),                         # more than 16 tokens
    # more than 16 tokens, one column tile per routed slot, shared experts: their gate/up and the
    # selection in the logits launch
    (dict(T=64, H=2048, E=64, I=1408, top_k=6, n_shared=2, I_shared=1408), 0, 1),
    (dict(T=40, E=32, top_k=2, n_shared=1, I_shared=64), 0, 1),
    (dict(T=40, E=16, top_k=6, n_shared=2, I_shared=64), 0, 0),   # four column tiles per slot
    (dict(T=4096, H=4096, E=8, I=14336, top_k=2), 0, 0),       # prefill
])
def test_forward_tables_pass_plan(m, kw, route_in_gateup, shared_in_router):
    t = m.moe_forward_tables(_shape(m, **kw))
    assert (t["route_in_gateup"], t["shared_in_router"]) == (route_in_gateup, shared_in_router)
