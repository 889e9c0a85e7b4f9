"""moe_forward_noalloc (the library's static scratch as workspace) against
moe_forward (a caller workspace) through the C ABI: two calls in a row on
each path, the second with a smaller input, each compared with moe_forward's
output on the same inputs (bit for bit: every path, the prefill combine
included, adds in a fixed order), and with the oracle to the usual
tolerance.  Also: shapes beyond
the scratch are rejected before anything runs, and a captured graph of the
call replays correctly."""
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return H.lib()


def _same(a, b, prefill):
    """Bit for bit on every path (prefill included: its combine adds in a fixed order)."""
    import torch
    va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
    vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
    return bool(torch.equal(va, vb))


def _noalloc(m, wl, t, path):
    import torch
    out = torch.full_like(t["x"], float("nan"))
    m.moe_forward_noalloc(H.shape_of(m, wl, path), t["x"], t["router_w"], t["router_b"], t["w_gate"], t["w_up"],
                          t["w_down"], t.get("ws_gate"), t.get("ws_up"), t.get("ws_down"), out)
    return out


# (larger, smaller) pairs: the second call reuses the scratch the first left behind
PAIRS = [
    (W("na_mixtral_t8", T=8, H=512, E=8, k=2, I=1024), W("na_mixtral_t3", T=3, H=512, E=8, k=2, I=1024), 1),
    (W("na_q4_t5", T=5, H=288, E=64, k=8, I=160, S=1, Is=96, x_dtype="f32", w_dtype="q4_0", r_dtype="f32"),
     W("na_q4_t1", T=1, H=256, E=64, k=8, I=128, S=1, Is=96, x_dtype="f32", w_dtype="q4_0", r_dtype="f32"), 0),
    (W("na_ds_t40", T=40, H=256, E=16, k=6, I=96, S=2, Is=160), W("na_ds_t8", T=8, H=256, E=16, k=6, I=96, S=2,
                                                                   Is=160), 0),
    (W("na_fused_t20", T=20, H=256, E=16, k=6, I=96, S=2, Is=160),
     W("na_fused_t5", T=5, H=256, E=16, k=6, I=96, S=2, Is=160), 3),
    (W("na_prefill_t300", T=300, H=352, E=8, k=2, I=416, S=1, Is=224, zipf_s=1.2),
     W("na_prefill_t130", T=130, H=256, E=8, k=2, I=256, S=1, Is=224, zipf_s=1.2), 2),
    (W("na_f32_t100", T=100, H=64, E=4, k=2, I=128, S=2, Is=64, x_dtype="f32", w_dtype="f32", r_dtype="f32"),
     W("na_f32_t4", T=4, H=64, E=4, k=2, I=128, x_dtype="f32", w_dtype="f32", r_dtype="f32"), 0),
]


@pytest.mark.parametrize("big, small, path", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_equals_moe_forward_twice(m, big, small, path):
    import torch
    for i, wl in enumerate((big, small)):
        inp = synth.make_inputs(wl, 20 + i)
        t = synth.to_torch(inp)
        got = _noalloc(m, wl, t, path)
        want = H.run_forward(m, wl, t, path=path)
        torch.cuda.synchronize()
        print(f"noalloc {wl.name} path={path} call {i + 1}", flush=True)
        assert _same(got, want, path == 2), (wl.name, i)
        err = H.relerr(H.to_f64(got), H.oracle_layer(wl, inp)["out"])
        assert err <= H.tolerance(wl), (wl.name, err)


def test_noalloc_rejects_shapes_beyond_the_scratch(m):
    wl = synth.WORKLOADS["mixtral_prefill_t4096"]
    shape = H.shape_of(m, wl)
    assert m.moe_workspace_size(shape) > m.MOE_NOALLOC_SCRATCH_BYTES
    rc = m.moe_forward_noalloc(shape, 16, 16, None, 16, 16, 16, None, None, None, 16, check=False)
    assert rc == m.MOE_ERR_TOO_LARGE


def test_noalloc_graph_replay(m):
    """Captured into a HIP graph (the caller that cannot allocate), replayed
    several times with eager work in between, each replay equal to eager."""
    import torch
    wl = W("na_graph_t8", T=8, H=256, E=16, k=6, I=96, S=2, Is=160)
    t = synth.to_torch(synth.make_inputs(wl, 30))
    shape = H.shape_of(m, wl)
    eager = _noalloc(m, wl, t, 0).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        m.moe_forward_noalloc(shape, t["x"], t["router_w"], t["router_b"], t["w_gate"], t["w_up"], t["w_down"],
                              t["ws_gate"], t["ws_up"], t["ws_down"], out, stream=cap.cuda_stream)
    for r in range(3):
        out.fill_(float("nan"))
        H.run_forward(m, wl, t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, eager, False), r
