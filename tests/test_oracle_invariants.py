"""Invariants and special cases that hold for the MoE layer whatever the weights.

Each one follows from the definition of the layer, not from the oracle's
code: identical experts reduce to one dense FFN; top_k = E is the full
softmax mixture; shared experts do not depend on the router; permuting
experts or tokens permutes the results; the layer is linear in the down
projections.  The last tests plant mistakes in the oracle (on the CPU) and
check that the pins catch them.
"""
import numpy as np
import pytest

import oracle
import oracle.moe as om
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(seed, T=6, H=16, E=5, I=12, S=0, Is=8, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((E, H)) * 0.4
    b = rng.standard_normal(E) if bias else None
    Wg = rng.standard_normal((E, I, H)) * 0.25
    Wu = rng.standard_normal((E, I, H)) * 0.25
    Wd = rng.standard_normal((E, H, I)) * 0.25
    sh = None
    if S:
        sh = (rng.standard_normal((S, Is, H)) * 0.25, rng.standard_normal((S, Is, H)) * 0.25,
              rng.standard_normal((S, H, Is)) * 0.25)
    return x, Wr, b, Wg, Wu, Wd, sh


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("k", [1, 2, 4])
def test_weights_sum_to_one_nonincreasing_distinct(seed, k):
    x, Wr, b, *_ = _rand(seed, T=20, E=7, bias=seed % 2 == 1)
    l, p, ids, w = oracle.route(x, Wr, b, k)
    assert np.allclose(w.sum(-1), 1.0, atol=1e-12, rtol=0)
    assert np.all(np.diff(w, axis=-1) <= 1e-15)
    for row in ids:
        assert len(set(row.tolist())) == k
    # the selected logits are the k largest
    kth = -np.sort(-l, axis=-1)[:, k - 1]
    assert np.all(np.take_along_axis(l, ids, -1) >= kth[:, None])


def test_bias_shift_invariance():
    x, Wr, b, Wg, Wu, Wd, _ = _rand(3, bias=True)
    r1 = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 2)
    r2 = oracle.moe_forward(x, Wr, b + 7.25, Wg, Wu, Wd, 2)
    assert (r1["ids"] == r2["ids"]).all()
    assert np.allclose(r1["out"], r2["out"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("k", [1, 2, 5])
def test_identical_experts_reduce_to_dense_ffn(k):
    x, Wr, _, Wg, Wu, Wd, _ = _rand(5)
    E = Wg.shape[0]
    G, U, D = (np.repeat(a[:1], E, axis=0) for a in (Wg, Wu, Wd))
    out = oracle.moe_forward(x, Wr, None, G, U, D, k)["out"]
    dense = oracle.swiglu_ffn(x, G[0], U[0], D[0])
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)


def test_single_expert_is_dense_ffn():
    x, Wr, _, Wg, Wu, Wd, _ = _rand(6, E=1)
    out = oracle.moe_forward(x, Wr, None, Wg, Wu, Wd, 1)["out"]
    assert np.allclose(out, oracle.swiglu_ffn(x, Wg[0], Wu[0], Wd[0]), rtol=1e-13, atol=1e-15)


def test_top_k_equal_E_is_full_softmax_mixture():
    """With k = E renormalisation is a no-op: out = sum_e p_e FFN_e(x), built here
    from the dense gate matrix and every expert applied to every token."""
    x, Wr, b, Wg, Wu, Wd, _ = _rand(7, bias=True)
    E = Wg.shape[0]
    r = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, E)
    assert np.allclose(r["w"].sum(-1), 1.0)
    p = oracle.softmax(oracle.router_logits(x, Wr, b))
    full = sum(p[:, e:e + 1] * oracle.swiglu_ffn(x, Wg[e], Wu[e], Wd[e]) for e in range(E))
    assert np.allclose(r["out"], full, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("k", [1, 3])
def test_gate_matrix_formulation(k):
    x, Wr, b, Wg, Wu, Wd, sh = _rand(8, S=1)
    r = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, k, sh)
    G = oracle.dense_gate_matrix(r["ids"], r["w"], Wg.shape[0])
    alt = sum(G[:, e:e + 1] * oracle.swiglu_ffn(x, Wg[e], Wu[e], Wd[e]) for e in range(Wg.shape[0]))
    alt = alt + oracle.swiglu_ffn(x, sh[0][0], sh[1][0], sh[2][0])
    assert np.allclose(r["out"], alt, rtol=1e-12, atol=1e-14)


def test_shared_expert_independent_of_router():
    x, Wr, b, Wg, Wu, Wd, sh = _rand(9, S=2)
    zero = np.zeros_like(Wd)
    r1 = oracle.moe_forward(x, Wr, b, Wg, Wu, zero, 2, sh)
    r2 = oracle.moe_forward(x, -Wr[::-1], b, Wg, Wu, zero, 2, sh)
    shared_only = sum(oracle.swiglu_ffn(x, sh[0][s], sh[1][s], sh[2][s]) for s in range(2))
    assert np.allclose(r1["out"], shared_only, rtol=1e-13, atol=1e-15)
    assert np.allclose(r2["out"], shared_only, rtol=1e-13, atol=1e-15)


def test_two_shared_experts_equal_one_of_double_width():
    x, Wr, b, Wg, Wu, Wd, sh = _rand(10, S=2, Is=6)
    one = (np.concatenate([sh[0][0], sh[0][1]], 0)[None], np.concatenate([sh[1][0], sh[1][1]], 0)[None],
           np.concatenate([sh[2][0], sh[2][1]], 1)[None])
    a = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 2, sh)["out"]
    c = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 2, one)["out"]
    assert np.allclose(a, c, rtol=1e-12, atol=1e-14)


def test_expert_permutation_symmetry():
    x, Wr, b, Wg, Wu, Wd, sh = _rand(11, bias=True, S=1)
    perm = np.array([3, 0, 4, 1, 2])
    r1 = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 2, sh)
    r2 = oracle.moe_forward(x, Wr[perm], b[perm], Wg[perm], Wu[perm], Wd[perm], 2, sh)
    inv = np.argsort(perm)
    assert (perm[r2["ids"]] == r1["ids"]).all()
    assert (r2["ids"] == inv[r1["ids"]]).all()
    assert np.allclose(r1["out"], r2["out"], rtol=1e-12, atol=1e-14)


def test_token_permutation_symmetry():
    x, Wr, b, Wg, Wu, Wd, sh = _rand(12, S=1)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    r1 = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 3, sh)
    r2 = oracle.moe_forward(x[perm], Wr, b, Wg, Wu, Wd, 3, sh)
    assert np.allclose(r1["out"][perm], r2["out"], rtol=1e-13, atol=1e-15)


def test_linear_in_down_projections():
    x, Wr, b, Wg, Wu, Wd, sh = _rand(13, S=1)
    c = -2.5
    r1 = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, 2, sh)["out"]
    sh2 = (sh[0], sh[1], c * sh[2])
    r2 = oracle.moe_forward(x, Wr, b, Wg, Wu, c * Wd, 2, sh2)["out"]
    assert np.allclose(c * r1, r2, rtol=1e-13, atol=1e-14)


def test_q4_codes_eight_give_zero_output():
    wl = synth.Workload("t", T=3, H=64, E=4, k=2, I=32, x_dtype="f32", w_dtype="q4_0", r_dtype="f32")
    rng = np.random.default_rng(0)
    q = np.full((4, 32, 64), 8, np.uint8)
    qd = np.full((4, 64, 32), 8, np.uint8)
    d1 = rng.random((4, 32, 2)).astype(np.float16)
    d2 = rng.random((4, 64, 1)).astype(np.float16)
    inp = dict(x=rng.standard_normal((3, 64)).astype(np.float32),
               router_w=rng.standard_normal((4, 64)).astype(np.float32), router_b=None,
               w_gate=synth.q4_0_pack(q, d1), w_up=synth.q4_0_pack(q, d1), w_down=synth.q4_0_pack(qd, d2))
    dec = oracle.decode_workload_inputs(inp, wl)
    r = oracle.moe_forward(dec["x"], dec["Wr"], None, dec["Wg"], dec["Wu"], dec["Wd"], 2)
    assert np.all(r["out"] == 0.0)


def test_generated_workload_decodes_and_runs():
    wl = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(wl, 0)
    dec = oracle.decode_workload_inputs(inp, wl)
    r = oracle.moe_forward(dec["x"], dec["Wr"], dec["b"], dec["Wg"], dec["Wu"], dec["Wd"], wl.k, dec["shared"])
    assert r["out"].shape == (wl.T, wl.H) and np.isfinite(r["out"]).all()
    # the generator is deterministic per seed
    inp2 = synth.make_inputs(wl, 0)
    assert all((inp[k2] == inp2[k2]).all() for k2 in ("x", "router_w", "w_gate", "w_up", "w_down"))


# ------------------------------------------------- planted mistakes (CPU) ---

@pytest.mark.parametrize("mutation", ["silu_sign", "transposed_up", "no_renorm", "drop_shared",
                                      "topk_ascending"])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutation):
    import tests.test_oracle_pins as pins
    if mutation == "silu_sign":
        monkeypatch.setattr(om, "silu", lambda z: z / (1.0 + np.exp(z)))
    elif mutation == "transposed_up":
        def bad(x, Wg, Wu, Wd):
            a = om.silu(x @ Wg.T) * (x @ Wg.T)    # up projection replaced by gate
            return a @ Wd.T
        monkeypatch.setattr(om, "swiglu_ffn", bad)
    elif mutation == "no_renorm":
        monkeypatch.setattr(om, "renormalize", lambda p, ids: np.take_along_axis(p, ids, -1))
    elif mutation == "drop_shared":
        orig_tokens = om.moe_forward_tokens
        monkeypatch.setattr(om, "moe_forward_tokens",
                            lambda x, ids, w, Wg, Wu, Wd, shared=None: orig_tokens(x, ids, w, Wg, Wu, Wd, None))
    elif mutation == "topk_ascending":
        monkeypatch.setattr(om, "select_topk",
                            lambda l, k: np.argsort(l, axis=-1, kind="stable")[:, :k])
    caught = 0
    for check in [pins.test_swiglu_closed_form, pins.test_router_closed_form,
                  pins.test_layer_closed_form_with_shared_expert]:
        try:
            check()
        except AssertionError:
            caught += 1
    for case in [dict(seed=0, T=3, H=5, E=4, k=2, I=6), dict(seed=2, T=2, H=7, E=3, k=3, I=5, S=1, Is=3)]:
        try:
            pins.test_vectorised_matches_brute_force(case)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"planted mistake {mutation} not caught"
