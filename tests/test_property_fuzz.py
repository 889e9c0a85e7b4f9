"""Property fuzz over random small shapes and seeds (hypothesis).

CPU: the vectorised fp64 oracle against the pure-Python brute force on
tiny layers of every shape the ABI admits at that size (tokens, hidden,
experts, top-k, intermediate, shared experts, router bias): outputs, expert
choice, weights and the expert-sorted order.

GPU: random small layers, each run on the paths its dtypes allow (automatic,
decode, prefill, single-launch decode) through the C ABI and compared with
the oracle to the usual bars.  The run is bounded (fixed seed, a fixed number
of examples, no shrinking, no example database) and stops at the first
failing example, which it prints.
"""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, Phase, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import loops  # noqa: E402
from tests import helpers as H  # noqa: E402

W = synth.Workload


# ---------------------------------------------------------------- CPU ----

@st.composite
def tiny_layer(draw):
    T = draw(st.integers(1, 5))
    Hd = draw(st.integers(1, 6))
    E = draw(st.integers(1, 6))
    k = draw(st.integers(1, E))
    I = draw(st.integers(1, 5))
    S = draw(st.integers(0, 2))
    Is = draw(st.integers(1, 4))
    bias = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return T, Hd, E, k, I, S, Is, bias, seed


@settings(max_examples=120, derandomize=True, deadline=None, database=None)
@given(tiny_layer())
def test_oracle_matches_brute_force(p):
    T, Hd, E, k, I, S, Is, bias, seed = p
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, Hd))
    Wr = rng.normal(0, 0.7, size=(E, Hd))
    b = rng.normal(size=E) if bias else None
    Wg, Wu, Wd = rng.normal(size=(E, I, Hd)), rng.normal(size=(E, I, Hd)), rng.normal(size=(E, Hd, I))
    sh = (rng.normal(size=(S, Is, Hd)), rng.normal(size=(S, Is, Hd)), rng.normal(size=(S, Hd, Is))) if S else None
    got = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, k, sh)
    want, ids, w = loops.moe_forward(x.tolist(), Wr.tolist(), None if b is None else b.tolist(), Wg.tolist(),
                                     Wu.tolist(), Wd.tolist(), k,
                                     None if sh is None else tuple(a.tolist() for a in sh))
    assert np.array_equal(got["ids"], np.array(ids))
    assert np.allclose(got["w"], np.array(w), rtol=1e-12, atol=1e-14)
    assert np.allclose(got["out"], np.array(want), rtol=1e-10, atol=1e-10)
    for M in (1, 3, 8):
        d, db = oracle.dispatch(got["ids"], E, M), loops.dispatch(ids, E, M)
        for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv", "active"):
            assert np.array_equal(d[key], np.array(db[key])), (M, key)


# ---------------------------------------------------------------- GPU ----

# (x, expert weights, router) dtype triples the ABI supports
DTYPES = [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("f32", "q4_0", "f32"), ("bf16", "q4_0", "bf16"),
          ("f32", "bf16", "bf16"), ("bf16", "q8_0", "bf16"), ("f32", "q8_0", "f32"), ("bf16", "fp8_e4m3", "bf16"),
          ("bf16", "f32", "f32")]


@st.composite
def small_layer(draw):
    x_dt, w_dt, r_dt = draw(st.sampled_from(DTYPES))
    bf16 = x_dt == "bf16" and w_dt == "bf16"
    T = draw(st.integers(0, 300 if bf16 else 90))
    Hd = 32 * draw(st.integers(1, 10))
    E = draw(st.integers(1, 80))
    k = draw(st.integers(1, min(E, 12)))
    I = 32 * draw(st.integers(1, 8))
    S = draw(st.integers(0, 2))
    Is = 32 * draw(st.integers(1, 6))
    zipf = draw(st.sampled_from([None, 1.2]))
    seed = draw(st.integers(0, 10 ** 6))
    paths = [0, 1]
    if bf16:
        paths.append(2)
    if r_dt == x_dt and k <= 16 and w_dt in ("f32", "bf16", "q4_0"):
        paths.append(3)
    path = draw(st.sampled_from(paths))
    wl = W(f"fuzz_T{T}_H{Hd}_E{E}_k{k}_I{I}_S{S}x{Is}_{x_dt}_{w_dt}_{r_dt}", T=T, H=Hd, E=E, k=k, I=I,
           S=S, Is=Is if S else 0, x_dtype=x_dt, w_dtype=w_dt, r_dtype=r_dt, zipf_s=zipf)
    return wl, seed, path


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return H.lib()


@pytest.mark.gpu
def test_gpu_layers_match_oracle(m):
    import torch
    count = [0]

    @settings(max_examples=150, derandomize=True, deadline=None, database=None,
              phases=[Phase.generate], suppress_health_check=list(HealthCheck))
    @given(small_layer())
    def run(p):
        wl, seed, path = p
        count[0] += 1
        print(f"fuzz case {count[0]}: {wl.name} seed={seed} path={path}", flush=True)
        inp = synth.make_inputs(wl, seed)
        t = synth.to_torch(inp)
        out = H.run_forward(m, wl, t, path=path)
        torch.cuda.synchronize()
        if wl.T == 0:
            return
        got = H.to_f64(out)
        r = H.run_route(m, wl, t)
        ref = H.oracle_layer(wl, inp)
        n_diff, _ = H.check_ids(r["topk_ids"], ref["logits"], wl.k)
        d = oracle.dispatch(r["topk_ids"].astype(np.int64), wl.E, r["tile_m"])
        for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv"):
            assert np.array_equal(r[key], d[key]), key
        if n_diff:
            ref = H.oracle_layer(wl, inp, ids=r["topk_ids"])
        assert np.isfinite(got).all()
        err = H.relerr(got, ref["out"])
        assert err <= H.tolerance(wl), (wl.name, seed, path, err)

    run()
    print(f"fuzz: {count[0]} layers matched the oracle", flush=True)
