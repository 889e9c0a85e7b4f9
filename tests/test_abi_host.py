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
    text = open(os.path.join(root, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


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
    the multi-launch decode of the same shape needs less."""
    fused = m.moe_workspace_size(m.make_shape(8, 4096, 8, 14336, 2, path=m.MOE_PATH_DECODE_FUSED))
    multi = m.moe_workspace_size(m.make_shape(8, 4096, 8, 14336, 2, path=m.MOE_PATH_DECODE))

    # work list: 4 logits planes, 1 selection, 8 x 896 gate/up tiles, 8 x 128 down row groups (32 outputs
    # each), 32 combine blocks
    n_items = 4 + 1 + 8 * 896 + 8 * 128 + 32
    assert fused - multi >= n_items * 8


def test_workspace_size_and_dims(m):
    s = m.make_shape(4096, 4096, 8, 14336, 2)
    tile_m, cap, n_tiles = m.moe_dispatch_dims(s)
    assert tile_m == 128 and cap == (4096 * 2 + 8 * 127 + 127) // 128 * 128 and n_tiles * tile_m == cap
    big = m.moe_workspace_size(s)
    # prefill needs the bf16 activations and the fp32 accumulator
    assert big >= cap * 14336 * 2 + 4096 * 4096 * 4
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
