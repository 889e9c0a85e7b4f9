"""GPU parity of the budgeted channel-sparse routed experts
(moe_forward_channel_sparse) against the fp64 oracle: per (token, engaged
expert) the c highest-scoring channels, the FFN over those channels only,
shared experts dense.

Small cases span several 16-channel tiles with ragged tails, several token
passes, ties and NaN among the scores, and the full budget (which is the
dense layer).  The full-size batch-one case is checked against the oracle
expert by expert.  Bars as for the dense layer: 1e-5 (fp32) or 1e-2 (bf16),
normwise."""
import numpy as np
import pytest

import oracle
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = {
    # name: (workload, budget)
    "bf16_t1_c182": (W("bf16_t1", T=1, H=256, E=8, k=2, I=1024), 182),
    "bf16_t5_shared_c37": (W("bf16_t5_shared", T=5, H=352, E=8, k=2, I=160, S=1, Is=96), 37),
    "bf16_t70_c40": (W("bf16_t70", T=70, H=128, E=8, k=2, I=96), 40),
    "f32_t3_c9": (W("f32_t3", T=3, H=96, E=4, k=2, I=64, x_dtype="f32", w_dtype="f32", r_dtype="f32"), 9),
    "bf16_full_budget": (W("bf16_full", T=4, H=256, E=4, k=2, I=128, S=1, Is=64), 128),
    "bf16_c1": (W("bf16_c1", T=2, H=192, E=6, k=3, I=64), 1),
    "bf16_wide_h_c300": (W("bf16_wide_h", T=2, H=4160, E=4, k=2, I=1536), 300),
    "f32x_bf16w_t8_c64": (W("f32x_bf16w", T=8, H=256, E=16, k=4, I=512, x_dtype="f32", r_dtype="bf16"), 64),
    "bf16_k10_c20": (W("bf16_k10", T=3, H=128, E=12, k=10, I=64), 20),
}


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return H.lib()


def _inputs(wl, seed, scores=None):
    inp = synth.make_inputs(wl, seed)
    inp["scores"] = synth.channel_scores(wl, seed) if scores is None else scores
    inp["w_down_t"] = synth.down_transposed(inp["w_down"], wl.E, wl.H, wl.I)
    return inp


def _run(m, wl, c, t, ws=None):
    import torch
    shape = H.shape_of(m, wl)
    if ws is None:
        ws = m.alloc_sparse_workspace(shape, c)
    out = torch.empty_like(t["x"])
    m.moe_forward_channel_sparse(shape, c, t["scores"], t["x"], t["router_w"], t["router_b"], t["w_gate"], t["w_up"],
                                 t["w_down_t"], t.get("ws_gate"), t.get("ws_up"), t.get("ws_down"), out, ws)
    return out


def _check(m, wl, c, inp):
    import torch
    t = synth.to_torch(inp)
    out = _run(m, wl, c, t)
    r = H.run_route(m, wl, t)
    torch.cuda.synchronize()
    dec = oracle.decode_workload_inputs(inp, wl)
    l = oracle.router_logits(dec["x"], dec["Wr"], dec["b"])
    n_diff, n_ties = H.check_ids(r["topk_ids"], l, wl.k)
    ids = r["topk_ids"].astype(np.int64) if n_diff else None
    ref = oracle.moe_forward_channel_sparse(dec["x"], dec["Wr"], dec["b"], dec["Wg"], dec["Wu"], dec["Wd"], wl.k,
                                            inp["scores"].astype(np.float64), c, dec["shared"], ids=ids)
    got = H.to_f64(out)
    err = H.relerr(got, ref["out"])
    print(f"{wl.name} c={c} relerr={err:.3e} near_ties={n_ties} differing={n_diff}", flush=True)
    assert np.isfinite(got).all()
    assert err <= H.tolerance(wl), err
    return got


@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_forward(m, name):
    wl, c = CASES[name]
    _check(m, wl, c, _inputs(wl, 1))


def test_sparse_score_ties_and_nan(m):
    """Equal scores keep the lower channel index; NaN scores rank below every number."""
    wl, c = CASES["bf16_t1_c182"]
    s = np.zeros((wl.T, wl.E, wl.I), dtype=np.float32)
    s[..., ::7] = np.nan
    s[..., 500:520] = 1.0
    _check(m, wl, c, _inputs(wl, 2, scores=s))


def test_full_budget_matches_dense_forward(m):
    import torch
    wl, c = CASES["bf16_full_budget"]
    inp = _inputs(wl, 3)
    t = synth.to_torch(inp)
    sparse = H.to_f64(_run(m, wl, c, t))
    dense = H.to_f64(H.run_forward(m, wl, t, path=1))
    torch.cuda.synchronize()
    assert H.relerr(sparse, dense) <= 1e-2


def test_sparse_deterministic_and_no_workspace_initialisation(m):
    import torch
    wl, c = CASES["bf16_t5_shared_c37"]
    t = synth.to_torch(_inputs(wl, 4))
    ws = m.alloc_sparse_workspace(H.shape_of(m, wl), c).fill_(0xA5)
    a = _run(m, wl, c, t, ws=ws).clone()
    ws.fill_(0x3C)
    b = _run(m, wl, c, t, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_full_size_batch_one(m):
    """Mixtral-shaped layer at batch one, 17.8 % of the channels: the oracle
    decodes only the two engaged experts."""
    import torch
    wl = synth.WORKLOADS["mixtral_decode_t1_sparse"]
    c = synth.channel_count(wl)
    t = synth.make_inputs_torch(wl, seed=0)
    t["scores"] = torch.from_numpy(synth.channel_scores(wl, 0)).cuda()
    t["w_down_t"] = t["w_down"].transpose(1, 2).contiguous()
    out = _run(m, wl, c, t)
    r = H.run_route(m, wl, t)
    torch.cuda.synchronize()
    x = H.to_f64(t["x"])
    l = oracle.router_logits(x, H.to_f64(t["router_w"]), None)
    H.check_ids(r["topk_ids"], l, wl.k)
    ids = r["topk_ids"].astype(np.int64)
    w = oracle.renormalize(oracle.softmax(l), ids)
    scores = t["scores"].cpu().numpy().astype(np.float64)
    ref = np.zeros((wl.T, wl.H))
    for j in range(wl.k):
        e = int(ids[0, j])
        Wg = H.expert_f64(t, "w_gate", wl, e, wl.E, wl.I, wl.H)
        Wu = H.expert_f64(t, "w_up", wl, e, wl.E, wl.I, wl.H)
        Wd = H.expert_f64(t, "w_down", wl, e, wl.E, wl.H, wl.I)
        chan = oracle.select_channels(scores[0, e], c)
        ref[0] += w[0, j] * oracle.masked_swiglu(x[0:1], Wg, Wu, Wd, chan)[0]
    err = H.relerr(H.to_f64(out), ref)
    print(f"mixtral_decode_t1_sparse c={c}: relerr {err:.3e}", flush=True)
    assert err <= 1e-2, err
