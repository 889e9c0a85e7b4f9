"""Pins of the budgeted top-c channel-sparse oracle (no GPU): closed forms
(the full budget is the dense layer; the kept set equals the dense FFN with
the other channels' down columns zeroed), brute force on tiny shapes,
symmetry under channel permutation, and the tie rule."""
import numpy as np
import pytest

import oracle
from oracle import loops


def _layer(rng, T=5, H=12, E=4, I=10, S=1, Is=6):
    x = rng.normal(size=(T, H))
    Wr = rng.normal(0, 0.5, size=(E, H))
    Wg = rng.normal(0, 0.3, size=(E, I, H))
    Wu = rng.normal(0, 0.3, size=(E, I, H))
    Wd = rng.normal(0, 0.3, size=(E, H, I))
    sh = (rng.normal(0, 0.3, size=(S, Is, H)), rng.normal(0, 0.3, size=(S, Is, H)),
          rng.normal(0, 0.3, size=(S, H, Is))) if S else None
    scores = rng.normal(size=(T, E, I))
    return x, Wr, Wg, Wu, Wd, sh, scores


def test_select_channels_hand_example():
    assert oracle.select_channels([0.5, 2.0, 2.0, -1.0, 3.0], 3).tolist() == [1, 2, 4]
    assert oracle.select_channels([0.5, 2.0, 2.0, -1.0, 3.0], 2).tolist() == [1, 4]   # tie: lower index
    assert oracle.select_channels(np.zeros(6), 4).tolist() == [0, 1, 2, 3]


def test_select_channels_nan_ranks_lowest():
    """NaN ranks below every number, -inf included; NaNs among themselves and
    equal numbers go to the lower index (hand-worked)."""
    nan, inf = float("nan"), float("inf")
    # the two numbers first (1 at index 1, 0 at index 3), then the NaN at the lower index
    assert oracle.select_channels([nan, 1.0, nan, 0.0], 3).tolist() == [0, 1, 3]
    assert oracle.select_channels([nan, 1.0, nan, 0.0], 2).tolist() == [1, 3]
    assert oracle.select_channels([nan, 1.0, nan, 0.0], 4).tolist() == [0, 1, 2, 3]
    # -inf is a number: it outranks every NaN
    assert oracle.select_channels([nan, -inf], 1).tolist() == [1]
    assert oracle.select_channels([-inf, nan, -inf], 2).tolist() == [0, 2]
    assert oracle.select_channels([nan, nan, nan], 2).tolist() == [0, 1]
    # +inf first, ties at +inf by index
    assert oracle.select_channels([1.0, inf, nan, inf], 2).tolist() == [1, 3]


@pytest.mark.parametrize("seed", range(4))
def test_select_channels_nan_matches_brute_force(seed):
    """The masked FFN with NaN and repeated scores equals the brute force,
    whose ranking spells the rule out per channel."""
    rng = np.random.default_rng(40 + seed)
    I, H = 11, 7
    x = rng.normal(size=H)
    Wg, Wu, Wd = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    scores = np.round(rng.normal(size=I), 1)
    scores[rng.choice(I, size=4, replace=False)] = np.nan
    scores[rng.choice(I, size=1)] = -np.inf
    for c in (1, 5, 8, I):
        want = loops.sparse_ffn_one(x.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist(), scores.tolist(), c)
        got = oracle.masked_swiglu(x[None], Wg, Wu, Wd, oracle.select_channels(scores, c))[0]
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), c


@pytest.mark.parametrize("seed", range(3))
def test_full_budget_is_the_dense_layer(seed):
    rng = np.random.default_rng(seed)
    x, Wr, Wg, Wu, Wd, sh, scores = _layer(rng)
    dense = oracle.moe_forward(x, Wr, None, Wg, Wu, Wd, 2, sh)["out"]
    sparse = oracle.moe_forward_channel_sparse(x, Wr, None, Wg, Wu, Wd, 2, scores, Wg.shape[1], sh)["out"]
    assert np.allclose(sparse, dense, rtol=1e-12, atol=1e-12)


def test_kept_set_equals_dense_ffn_with_other_down_columns_zeroed():
    rng = np.random.default_rng(7)
    x, Wr, Wg, Wu, Wd, sh, scores = _layer(rng, S=0)
    c = 3
    l, p, ids, w = oracle.route(x, Wr, None, 2)
    got = oracle.moe_forward_channel_sparse(x, Wr, None, Wg, Wu, Wd, 2, scores, c)["out"]
    want = np.zeros_like(got)
    for t in range(x.shape[0]):
        for j in range(2):
            e = ids[t, j]
            keep = np.argsort(-scores[t, e], kind="stable")[:c]
            Wd_m = np.zeros_like(Wd[e])
            Wd_m[:, keep] = Wd[e][:, keep]
            want[t] += w[t, j] * oracle.swiglu_ffn(x[t:t + 1], Wg[e], Wu[e], Wd_m)[0]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("c", [1, 4, 9])
def test_masked_ffn_matches_brute_force(c):
    rng = np.random.default_rng(c)
    x, _, Wg, Wu, Wd, _, scores = _layer(rng, T=2, S=0)
    for t in range(2):
        for e in range(Wg.shape[0]):
            chan = oracle.select_channels(scores[t, e], c)
            v = oracle.masked_swiglu(x[t:t + 1], Wg[e], Wu[e], Wd[e], chan)[0]
            b = loops.sparse_ffn_one(list(x[t]), Wg[e].tolist(), Wu[e].tolist(), Wd[e].tolist(),
                                     list(scores[t, e]), c)
            assert np.allclose(v, b, rtol=1e-12, atol=1e-14)


def test_channel_permutation_symmetry():
    rng = np.random.default_rng(11)
    x, Wr, Wg, Wu, Wd, sh, scores = _layer(rng)
    perm = rng.permutation(Wg.shape[1])
    # distinct scores so that the kept set does not depend on index order
    scores = scores + 1e-9 * np.arange(scores.shape[2])
    a = oracle.moe_forward_channel_sparse(x, Wr, None, Wg, Wu, Wd, 2, scores, 4, sh)["out"]
    b = oracle.moe_forward_channel_sparse(x, Wr, None, Wg[:, perm], Wu[:, perm], Wd[:, :, perm], 2,
                                          scores[:, :, perm], 4, sh)["out"]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_planted_mistakes_are_caught():
    """A wrong kept set (lowest scores) or a dropped routing weight changes the result."""
    rng = np.random.default_rng(5)
    x, Wr, Wg, Wu, Wd, sh, scores = _layer(rng, S=0)
    good = oracle.moe_forward_channel_sparse(x, Wr, None, Wg, Wu, Wd, 2, scores, 4)["out"]
    flipped = oracle.moe_forward_channel_sparse(x, Wr, None, Wg, Wu, Wd, 2, -scores, 4)["out"]
    assert not np.allclose(good, flipped)
    l, p, ids, w = oracle.route(x, Wr, None, 2)
    unweighted = np.zeros_like(good)
    for t in range(x.shape[0]):
        for j in range(2):
            e = ids[t, j]
            unweighted[t] += oracle.masked_swiglu(x[t:t + 1], Wg[e], Wu[e], Wd[e],
                                                  oracle.select_channels(scores[t, e], 4))[0]
    assert not np.allclose(good, unweighted)
