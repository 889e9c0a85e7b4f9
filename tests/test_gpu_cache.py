"""GPU: host-resident experts behind a GPU expert cache with prefetching
("FATE: how to speed up MoE inference in llama.cpp with an expert cache and
prefetching", ai-manual.ru, sections "How the expert cache works" and
"Predictive prefetching: guessing the future").

The routed experts of several layers live in pinned host memory and a cache
of fewer slots than one layer has experts serves them; an expert that is not
resident is read from host memory by the kernels themselves.  Every call's
output must be within the oracle's tolerance, equal bit for bit to the same
call through a cache that never evicts (where an expert is read from changes
no arithmetic), and equal up to the order of the fp32 sums to moe_forward
with the weights on the device.  The counters must add up, and prefetching by
the pages' rule (experts e + 1 in the next layer) must turn the next layer's
lookups into hits.
"""
import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload
WT_KEYS = ("w_gate", "w_up", "w_down")


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return H.lib()


def _pinned(a):
    """A new pinned host copy of a stored-bits numpy array (as bytes)."""
    import torch
    b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    t = torch.empty(b.size, dtype=torch.uint8, pin_memory=True)
    t.numpy()[:] = b
    return t


class Layers:
    """n_layers layers of one shape: numpy inputs, pinned host expert stacks,
    device copies of everything (for moe_forward) and device router/shared weights."""

    def __init__(self, wl, n_layers, seed, biases=None):
        self.wl = wl
        self.np = []
        for l in range(n_layers):
            inp = synth.make_inputs(wl, seed + l)
            if biases is not None:
                inp["router_b"] = np.asarray(biases[l], np.float32)
            self.np.append(inp)
        self.host = [tuple(_pinned(inp[k]) for k in WT_KEYS) for inp in self.np]
        self.dev = [synth.to_torch(inp) for inp in self.np]

    def x_for(self, call_seed):
        """The x of one call (same recipe as the layer inputs), numpy and torch."""
        x = synth.make_inputs(self.wl, 1000 + call_seed)["x"]
        return x, synth.to_torch({"x": x})["x"]


def _cache(m, layers, n_slots, depth=1, shift=1):
    import torch
    shape = H.shape_of(m, layers.wl, 1)
    region = torch.empty(m.moe_cache_region_bytes(shape, len(layers.host), n_slots), dtype=torch.uint8,
                         device="cuda")
    copy = torch.cuda.Stream()
    h = m.moe_cache_create(shape, layers.host, region, n_slots, depth, shift, copy)
    return dict(h=h, region=region, copy=copy, shape=shape)


def _cached_call(m, c, layers, l, x):
    import torch
    t = layers.dev[l]
    shape = H.shape_of(m, layers.wl, 1)
    ws = m.alloc_workspace(shape)
    out = torch.empty_like(x)
    m.moe_forward_cached(c["h"], l, shape, x, t["router_w"], t["router_b"], t.get("ws_gate"), t.get("ws_up"),
                         t.get("ws_down"), out, ws)
    return out


def _resident_call(m, layers, l, x):
    t = dict(layers.dev[l])
    t["x"] = x
    return H.run_forward(m, layers.wl, t, path=1)


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _destroy(m, c):
    import torch
    torch.cuda.synchronize()
    m.moe_cache_destroy(c["h"])


CASES = {
    # one token (the one-work-group down projection), a shared expert of the same size
    "bf16_t1": W("cache_bf16_t1", T=1, H=256, E=16, k=4, I=128, S=1, Is=128),
    "q4_t1": W("cache_q4_t1", T=1, H=256, E=16, k=4, I=128, S=1, Is=128, x_dtype="f32", w_dtype="q4_0",
               r_dtype="f32"),
    "q8_t1": W("cache_q8_t1", T=1, H=256, E=16, k=4, I=160, S=1, Is=160, w_dtype="q8_0"),
    "fp8_t3": W("cache_fp8_t3", T=3, H=256, E=16, k=2, I=192, S=1, Is=96, w_dtype="fp8_e4m3"),
    "f32_t2": W("cache_f32_t2", T=2, H=128, E=12, k=3, I=96, x_dtype="f32", w_dtype="f32", r_dtype="f32"),
}
N_SLOTS = {"bf16_t1": 6, "q4_t1": 5, "q8_t1": 6, "fp8_t3": 7, "f32_t2": 7}


@pytest.mark.parametrize("name", sorted(CASES))
def test_cached_layers_match_oracle_and_resident(m, name):
    import torch
    wl = CASES[name]
    L = 3
    layers = Layers(wl, L, seed=40)
    small = _cache(m, layers, N_SLOTS[name])
    big = _cache(m, layers, L * wl.E, depth=0)      # never evicts
    total_active = 0
    try:
        for call in range(9):
            l = call % L
            x_np, x = layers.x_for(call)
            got = _cached_call(m, small, layers, l, x)
            ref_big = _cached_call(m, big, layers, l, x)
            ref_dev = _resident_call(m, layers, l, x)
            torch.cuda.synchronize()
            assert torch.equal(_bits(got), _bits(ref_big)), (name, call)
            assert H.same_up_to_rounding(got, ref_dev), (name, call)
            inp = dict(layers.np[l])
            inp["x"] = x_np
            ref = H.oracle_layer(wl, inp)
            total_active += len(np.unique(ref["ids"]))
            err = H.relerr(H.to_f64(got), ref["out"])
            print(f"{name} call {call} layer {l} relerr={err:.3e}", flush=True)
            assert err <= H.tolerance(wl), (name, call, err)
        st = m.moe_cache_stats(small["h"])
        print(name, st, flush=True)
        assert st["lookups"] == total_active
        assert st["hits"] + st["misses"] == st["lookups"]
        assert st["misses"] > 0 and st["prefetches"] > 0
        assert st["prefetch_hits"] <= st["hits"]
    finally:
        _destroy(m, small)
        _destroy(m, big)


def test_prefetch_by_the_shift_rule_turns_misses_into_hits(m):
    """Layer 0 routes to experts 3 and 7, layer 1 to 4 and 8 (router biases):
    with depth 1 and shift 1 the call on layer 0 prefetches exactly what the
    call on layer 1 needs."""
    import torch
    wl = W("cache_prefetch", T=1, H=128, E=16, k=2, I=64)
    b0 = np.zeros(16, np.float32)
    b0[[3, 7]] = 30.0
    b1 = np.zeros(16, np.float32)
    b1[[4, 8]] = 30.0
    layers = Layers(wl, 2, seed=5, biases=[b0, b1])
    c = _cache(m, layers, 6, depth=1, shift=1)
    try:
        x_np, x = layers.x_for(0)
        _cached_call(m, c, layers, 0, x)
        torch.cuda.synchronize()
        s0 = m.moe_cache_stats(c["h"], reset=True)
        assert (s0["lookups"], s0["misses"], s0["prefetches"]) == (2, 2, 2), s0
        got = _cached_call(m, c, layers, 1, x)
        ref = _resident_call(m, layers, 1, x)
        torch.cuda.synchronize()
        s1 = m.moe_cache_stats(c["h"], reset=True)
        assert (s1["lookups"], s1["hits"], s1["prefetch_hits"], s1["misses"]) == (2, 2, 2, 0), s1
        assert H.same_up_to_rounding(got, ref)
        inp = dict(layers.np[1])
        inp["x"] = x_np
        r = H.oracle_layer(wl, inp)
        assert sorted(r["ids"][0].tolist()) == [4, 8]
        assert H.relerr(H.to_f64(got), r["out"]) <= H.tolerance(wl)
        # flushed: the same call misses again, and its output does not change
        m.moe_cache_flush(c["h"])
        again = _cached_call(m, c, layers, 1, x)
        torch.cuda.synchronize()
        s2 = m.moe_cache_stats(c["h"], reset=True)
        assert s2["misses"] == 2 and s2["hits"] == 0, s2
        assert torch.equal(_bits(again), _bits(got))
    finally:
        _destroy(m, c)


def test_two_passes_through_a_cache_smaller_than_the_layers(m):
    """70 tokens make two decode passes of 64 and 6; the cache holds one
    layer's experts, so every other call evicts the previous layer's."""
    import torch
    wl = W("cache_t70", T=70, H=128, E=8, k=2, I=64, S=1, Is=64)
    layers = Layers(wl, 2, seed=11)
    c = _cache(m, layers, 8, depth=1, shift=0)
    try:
        for call in range(4):
            l = call % 2
            x_np, x = layers.x_for(call)
            got = _cached_call(m, c, layers, l, x)
            ref = _resident_call(m, layers, l, x)
            torch.cuda.synchronize()
            assert torch.equal(_bits(got), _bits(ref)), call
            inp = dict(layers.np[l])
            inp["x"] = x_np
            r = H.oracle_layer(wl, inp)
            assert H.relerr(H.to_f64(got), r["out"]) <= H.tolerance(wl)
        st = m.moe_cache_stats(c["h"])
        assert st["hits"] + st["misses"] == st["lookups"] and st["misses"] >= 8
    finally:
        _destroy(m, c)


def test_cache_argument_errors(m):
    import torch
    wl = W("cache_err", T=1, H=128, E=16, k=4, I=64)
    layers = Layers(wl, 2, seed=3)
    shape = H.shape_of(m, wl, 1)
    region = torch.empty(m.moe_cache_region_bytes(shape, 2, 3), dtype=torch.uint8, device="cuda")
    copy = torch.cuda.Stream()
    # pageable host stacks are refused
    pageable = [tuple(torch.from_numpy(np.ascontiguousarray(inp[k]).view(np.uint8).reshape(-1)) for k in WT_KEYS)
                for inp in layers.np]
    assert m.moe_cache_create(shape, pageable, region, 3, 1, 1, copy, check=False) == m.MOE_ERR_NOT_PINNED
    # a region smaller than the slots need, a prefetch depth of n_layers
    assert m.moe_cache_create(shape, layers.host, region, 4, 1, 1, copy, check=False) == m.MOE_ERR_WORKSPACE
    assert m.moe_cache_create(shape, layers.host, region, 3, 2, 1, copy, check=False) == m.MOE_ERR_SHAPE
    h = m.moe_cache_create(shape, layers.host, region, 3, 1, 1, copy)
    try:
        t = layers.dev[0]
        ws = m.alloc_workspace(shape)
        out = torch.full_like(t["x"], 7.0)
        other = H.shape_of(m, wl.replace(I=96), 1)
        assert m.moe_forward_cached(h, 0, other, t["x"], t["router_w"], t["router_b"], None, None, None, out, ws,
                                    check=False) == m.MOE_ERR_SHAPE
        assert m.moe_forward_cached(h, 2, shape, t["x"], t["router_w"], t["router_b"], None, None, None, out, ws,
                                    check=False) == m.MOE_ERR_SHAPE
        torch.cuda.synchronize()
        assert (out == 7.0).all()
        assert m.moe_cache_stats(h)["lookups"] == 0
        # a token engages 4 experts and the cache has 3 slots: the rest are read from host memory
        for call in range(3):
            x_np, x = layers.x_for(call)
            got = _cached_call(m, {"h": h}, layers, call % 2, x)
            ref = _resident_call(m, layers, call % 2, x)
            torch.cuda.synchronize()
            assert H.same_up_to_rounding(got, ref)
        st = m.moe_cache_stats(h)
        assert st["lookups"] == 12 and st["hits"] + st["misses"] == 12
    finally:
        torch.cuda.synchronize()
        m.moe_cache_destroy(h)
