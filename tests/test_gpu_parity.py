"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases use numpy-drawn inputs whose stored bits both sides read; they
span several tiles with ragged tails and the edge cases of the method.  The
full-size workloads use torch-drawn inputs on the GPU (the same tensors are
copied to the host for the oracle), run in the launch configuration that
bench.py times, and are checked on sampled tokens the oracle computes one by
one, plus properties that hold at any size.

Bars: expert ids and the expert-sorted order bit-exact (tokens whose top-k
logits are within 1e-4 of a tie may pick either valid order); outputs within
a normwise relative error of 1e-5 (fp32 everywhere) or 1e-2 (bf16 or Q4_0).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

W = synth.Workload
SMALL = {
    "tiny_f32": synth.WORKLOADS["tiny_f32"],
    "mixtral_small_bf16": W("mixtral_small_bf16", T=8, H=512, E=8, k=2, I=1024),
    "qwen_small_q4_t1": W("qwen_small_q4_t1", T=1, H=256, E=64, k=8, I=128, S=1, Is=96,
                          x_dtype="f32", w_dtype="q4_0", r_dtype="f32"),
    "qwen_small_q4_t5": W("qwen_small_q4_t5", T=5, H=288, E=64, k=8, I=160, S=1, Is=96,
                          x_dtype="f32", w_dtype="q4_0", r_dtype="f32"),
    "deepseek_small_t8": W("deepseek_small_t8", T=8, H=256, E=16, k=6, I=96, S=2, Is=160),
    "deepseek_small_t40": W("deepseek_small_t40", T=40, H=256, E=16, k=6, I=96, S=2, Is=160),
    "prefill_small_zipf": W("prefill_small_zipf", T=300, H=352, E=8, k=2, I=416, S=1, Is=224, zipf_s=1.2),
    "x_f32_w_bf16_e5": W("x_f32_w_bf16_e5", T=6, H=192, E=5, k=3, I=160, x_dtype="f32", r_dtype="bf16"),
    "w_f32_x_bf16": W("w_f32_x_bf16", T=3, H=128, E=4, k=1, I=64, x_dtype="bf16", w_dtype="f32", r_dtype="f32"),
    "k_equals_E": W("k_equals_E", T=4, H=128, E=8, k=8, I=64),
    "q4_bf16x_t70": W("q4_bf16x_t70", T=70, H=128, E=8, k=2, I=64, w_dtype="q4_0"),
    "f32_t100_shared": W("f32_t100_shared", T=100, H=64, E=4, k=2, I=128, S=2, Is=64,
                         x_dtype="f32", w_dtype="f32", r_dtype="f32"),
    "t1_k1": W("t1_k1", T=1, H=96, E=3, k=1, I=32),
    "e20_k12": W("e20_k12", T=6, H=128, E=20, k=12, I=64),
    "e256_k70": W("e256_k70", T=3, H=64, E=256, k=70, I=32),
    # more assignments than the router keeps in LDS: the dispatch reads the ids back from memory
    "n10k_prefill": W("n10k_prefill", T=5000, H=64, E=8, k=2, I=32),
    # 33..64 experts (one DPP row per token) with k > 8 and a ragged expert count
    "e40_k10": W("e40_k10", T=37, H=96, E=40, k=10, I=64),
    # few assignments (the rank top-k and one-wave dispatch): one token over 256 experts, and
    # exactly 64 assignments over 32 experts
    "e256_t1_k8": W("e256_t1_k8", T=1, H=64, E=256, k=8, I=32),
    "n64_e32": W("n64_e32", T=8, H=64, E=32, k=8, I=32, S=1, Is=32),
    # two groups of experts per token, the second holding 8 (survivor slots left empty)
    "e72_t3_k6": W("e72_t3_k6", T=3, H=96, E=72, k=6, I=32, S=1, Is=32),
    # more than 16 tokens with few per expert: one-column-tile kernels with extra passes (the shared
    # slot takes three)
    "e32_t40_passes": W("e32_t40_passes", T=40, H=160, E=32, k=2, I=96, S=1, Is=64),
    # down work-groups of four row tiles (the grid keeps >= 2048 of them), with and without passes
    "rpw4_t16": W("rpw4_t16", T=16, H=1024, E=128, k=8, I=64),
    "rpw4_t24_passes": W("rpw4_t24_passes", T=24, H=2048, E=128, k=4, I=64, S=1, Is=64),
    # 8-bit expert weights: Q8_0 blocks with a partly filled last step (9 and 5 blocks per row),
    # fp8 rows whose length is 32 past a multiple of 64 (a half-filled last step)
    "q8_small_t5": W("q8_small_t5", T=5, H=288, E=64, k=8, I=160, S=1, Is=96,
                     x_dtype="f32", w_dtype="q8_0", r_dtype="f32"),
    "q8_bf16x_t40": W("q8_bf16x_t40", T=40, H=256, E=16, k=6, I=96, S=2, Is=160, w_dtype="q8_0"),
    "q8_f32_t70": W("q8_f32_t70", T=70, H=128, E=8, k=2, I=64, x_dtype="f32", w_dtype="q8_0", r_dtype="f32"),
    "fp8_small_t8": W("fp8_small_t8", T=8, H=512, E=8, k=2, I=1024, w_dtype="fp8_e4m3"),
    "fp8_tails_t40": W("fp8_tails_t40", T=40, H=352, E=16, k=6, I=96, S=2, Is=160, w_dtype="fp8_e4m3"),
    "fp8_f32x_t3": W("fp8_f32x_t3", T=3, H=96, E=5, k=2, I=64, x_dtype="f32", w_dtype="fp8_e4m3",
                     r_dtype="f32"),
    # prefill down GEMM with its k range split in two (K = 2048) and in four (K = 4096): the
    # shared expert's own K is cut into four ranges too, which leaves two of them empty (96 =
    # 64 + 32, the second half-full) or ragged with a half-full last stage (2080 = 576 + 576 +
    # 576 + 352)
    "prefill_ksplit2": W("prefill_ksplit2", T=300, H=256, E=4, k=2, I=2048, zipf_s=1.2),
    "prefill_ksplit4_shared": W("prefill_ksplit4_shared", T=290, H=256, E=4, k=2, I=4096, S=1, Is=96),
    "prefill_ksplit4_ragged": W("prefill_ksplit4_ragged", T=333, H=224, E=5, k=2, I=4096, S=1, Is=2080),
    # decode down projection with its reduction cut into two k ranges, summed in the down
    # launch's combine epilogue; with a shared expert whose shorter K splits unevenly (35 steps),
    # and with more than 16 slots (a combine launch of its own) and shared experts whose K of 3
    # steps leaves one range a single step
    "dn_ks2_t8": W("dn_ks2_t8", T=8, H=256, E=8, k=2, I=2048),
    "dn_ks2_shared_t5": W("dn_ks2_shared_t5", T=5, H=256, E=8, k=2, I=4096, S=1, Is=1120),
    "dn_ks2_wide_t8": W("dn_ks2_wide_t8", T=8, H=256, E=32, k=4, I=4096, S=2, Is=96),
    # one token whose slots share one K: the down projection adds every slot of a row group in one
    # work-group (Q4_0 and Q8_0 with a shared expert, bf16 with two steps per wave, fp32 with
    # uneven steps per wave), and one with more (slot, step) pairs than a wave holds, which keeps
    # the partial rows and the combine
    "t1_one_q4_shared": W("t1_one_q4_shared", T=1, H=288, E=64, k=8, I=128, S=1, Is=128,
                          x_dtype="f32", w_dtype="q4_0", r_dtype="f32"),
    "t1_one_q8_shared": W("t1_one_q8_shared", T=1, H=160, E=32, k=6, I=160, S=2, Is=160, w_dtype="q8_0"),
    "t1_one_bf16_2steps": W("t1_one_bf16_2steps", T=1, H=224, E=16, k=4, I=256, S=2, Is=256),
    "t1_one_f32": W("t1_one_f32", T=1, H=96, E=6, k=2, I=96, S=1, Is=96,
                    x_dtype="f32", w_dtype="f32", r_dtype="f32"),
    "t1_pairs_over": W("t1_pairs_over", T=1, H=128, E=32, k=8, I=256, S=2, Is=256),
    # down projection with each k range cut over eight waves (grids of >= 2048 two-row-tile work-groups):
    # 16 slots with the combine in the down epilogue, and 33 slots (a shared expert) with column passes
    # and a combine launch
    "dn_w8_epi_t8": W("dn_w8_epi_t8", T=8, H=4096, E=16, k=2, I=128),
    "dn_w8_passes_t32": W("dn_w8_passes_t32", T=32, H=2048, E=32, k=2, I=128, S=1, Is=128),
    # four 16-token column tiles with the combine in the down epilogue (9 slots): output row groups
    # of 16 (64 bytes), two to a 128-byte line, 10 of them (lines shared across work-groups)
    "epi_nct4_h160_t40": W("epi_nct4_h160_t40", T=40, H=160, E=8, k=2, I=64, S=1, Is=64),
}
BF16_BOTH_PATHS = ["mixtral_small_bf16", "deepseek_small_t8", "deepseek_small_t40", "prefill_small_zipf",
                   "k_equals_E", "t1_k1", "prefill_ksplit2", "prefill_ksplit4_shared", "prefill_ksplit4_ragged"]


@pytest.fixture(scope="module")
def m():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return H.lib()


def _inputs(wl, seed, bias=None):
    inp = synth.make_inputs(wl, seed)
    if bias is not None:
        inp["router_b"] = np.asarray(bias, dtype=np.float32)
    return inp


def _check_forward(m, wl, inp, path=0):
    import torch
    t = synth.to_torch(inp)
    out = H.run_forward(m, wl, t, path=path)
    r = H.run_route(m, wl, t)
    torch.cuda.synchronize()
    got = H.to_f64(out)
    ref = H.oracle_layer(wl, inp)
    n_diff, n_ties = H.check_ids(r["topk_ids"], ref["logits"], wl.k)
    if n_diff:
        ref = H.oracle_layer(wl, inp, ids=r["topk_ids"])
    err = H.relerr(got, ref["out"])
    print(f"{wl.name} path={path} seed-case relerr={err:.3e} near_ties={n_ties} differing={n_diff}", flush=True)
    assert np.isfinite(got).all()
    assert err <= H.tolerance(wl), err
    return got, ref


@pytest.mark.parametrize("seed", range(5))
def test_tiny_f32_all_seeds(m, seed):
    wl = SMALL["tiny_f32"]
    _check_forward(m, wl, _inputs(wl, seed))


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_auto_path(m, name):
    wl = SMALL[name]
    _check_forward(m, wl, _inputs(wl, 1))


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("name", BF16_BOTH_PATHS)
def test_forward_forced_paths(m, name, path):
    wl = SMALL[name]
    _check_forward(m, wl, _inputs(wl, 2), path=path)


def _fused_ok(wl):
    return wl.r_dtype == wl.x_dtype and wl.k <= 16 and wl.w_dtype in ("f32", "bf16", "q4_0")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_multi_launch_decode(m, name):
    wl = SMALL[name]
    _check_forward(m, wl, _inputs(wl, 8), path=1)


@pytest.mark.parametrize("name", sorted(n for n in SMALL if _fused_ok(SMALL[n])))
def test_single_launch_decode_matches_multi_launch(m, name):
    """The single-launch decode runs the same work items in one resident-grid
    launch, with handoffs through device-scope stores and flags: its output
    must be within the oracle's tolerance and equal to the multi-launch
    decode up to the order of the fp32 sums (the multi-launch down
    projection may cut its reduction into k ranges)."""
    import torch
    wl = SMALL[name]
    inp = _inputs(wl, 9)
    t = synth.to_torch(inp)
    multi = H.run_forward(m, wl, t, path=1)
    fused = H.run_forward(m, wl, t, path=3)
    torch.cuda.synchronize()
    assert H.same_up_to_rounding(fused, multi)
    _check_forward(m, wl, inp, path=3)


@pytest.mark.parametrize("H_", [128, 160])
def test_prefill_tile_classes(m, H_):
    """Expert counts chosen at the prefill row-tile boundaries: 129 rows (one
    full tile, 127 padding), 128 (a half tile: at most 128 rows in use), 385
    (a full tile, then a last tile of 129 rows), exactly 256 (no padding) and
    1 (a half tile of one row).  The routing is forced through one-hot router
    rows; H = 160 also leaves a half-full last k stage."""
    counts = [129, 128, 385, 256, 1]
    E = len(counts)
    T = sum(counts)
    wl = W("prefill_tiles", T=T, H=H_, E=E, k=1, I=96, S=1, Is=64)
    inp = _inputs(wl, 4)
    choice = np.repeat(np.arange(E), counts)
    np.random.default_rng(5).shuffle(choice)
    x = np.random.default_rng(6).standard_normal((T, H_)).astype(np.float32)
    x[:, :E] = 0.0
    x[np.arange(T), choice] = 4.0
    wr = np.zeros((E, H_), np.float32)
    wr[np.arange(E), np.arange(E)] = 1.0
    inp["x"] = synth.f32_to_bf16_bits(x)
    inp["router_w"] = synth.f32_to_bf16_bits(wr)
    inp["router_b"] = None
    _, ref = _check_forward(m, wl, inp, path=2)
    assert (ref["ids_used"][:, 0] == choice).all()
    assert np.bincount(ref["ids_used"][:, 0], minlength=E).tolist() == counts


@pytest.mark.parametrize("path", [1, 2, 3])
def test_all_tokens_to_one_expert(m, path):
    wl = W("one_expert", T=20, H=128, E=8, k=2, I=64, S=1, Is=64)
    bias = np.zeros(8, np.float32)
    bias[3] = 30.0
    _, ref = _check_forward(m, wl, _inputs(wl, 3, bias), path=path)
    assert (ref["ids_used"][:, 0] == 3).all()


def test_empty_batch_is_noop(m):
    import torch
    wl = SMALL["mixtral_small_bf16"].replace(T=0)
    shape = H.shape_of(m, wl)
    ws = m.alloc_workspace(shape)
    x = torch.empty(0, wl.H, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    assert m.moe_forward(shape, x, w, None, w, w, w, None, None, None, x, ws) == 0


@pytest.mark.parametrize("name", ["mixtral_small_bf16", "qwen_small_q4_t5", "deepseek_small_t40",
                                  "prefill_small_zipf", "k_equals_E", "tiny_f32", "e20_k12", "e256_k70",
                                  "n10k_prefill", "e40_k10", "e256_t1_k8", "n64_e32", "qwen_small_q4_t1",
                                  "t1_k1", "e72_t3_k6"])
def test_route_bit_exact(m, name):
    wl = SMALL[name]
    inp = _inputs(wl, 4)
    t = synth.to_torch(inp)
    r = H.run_route(m, wl, t)
    dec = oracle.decode_workload_inputs(inp, wl)
    l, p, ids_o, w_o = oracle.route(dec["x"], dec["Wr"], dec["b"], wl.k)
    H.check_ids(r["topk_ids"], l, wl.k)
    w_ref = oracle.renormalize(p, r["topk_ids"].astype(np.int64))
    assert np.allclose(r["topk_w"], w_ref, rtol=2e-6, atol=1e-7)
    d = oracle.dispatch(r["topk_ids"].astype(np.int64), wl.E, r["tile_m"])
    for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv"):
        assert np.array_equal(r[key], d[key]), key
    act = r["active"]
    assert act[0] == len(d["active"]) and np.array_equal(act[1:1 + act[0]], d["active"])


def _forward_tables(m, wl, t, path, ws):
    """Run moe_forward and read the routing of its last pass from the workspace."""
    import torch
    shape = H.shape_of(m, wl, path)
    H.run_forward(m, wl, t, path=path, ws=ws)
    torch.cuda.synchronize()
    L = m.moe_forward_tables(shape)
    n = L["tokens"] * wl.k

    def arr(key, count, dtype=torch.int32):
        o = L[key]
        return ws[o:o + 4 * count].view(dtype).cpu().numpy()
    r = dict(topk_ids=arr("topk_ids", n).reshape(-1, wl.k), topk_w=arr("topk_w", n, torch.float32).reshape(-1, wl.k),
             counts=arr("counts", wl.E), offsets=arr("offsets", wl.E + 1), sorted_ids=arr("sorted_ids", L["capacity"]),
             inv=arr("inv", n), active=arr("active", wl.E + 1))
    if L["n_tiles"]:
        r["tile_expert"] = arr("tile_expert", L["n_tiles"])
    return L, r


# (case, path): decode with the routing in the gate/up prologue (few assignments), with a
# separate selection launch, several passes (the tables hold the last one), the single
# launch with and without a selection item, and prefill (256-row padding)
TABLE_CASES = [("qwen_small_q4_t1", 1), ("e256_t1_k8", 1), ("deepseek_small_t8", 1), ("deepseek_small_t40", 1),
               ("q4_bf16x_t70", 1), ("f32_t100_shared", 1), ("e40_k10", 1), ("deepseek_small_t8", 3),
               ("deepseek_small_t40", 3), ("qwen_small_q4_t1", 3), ("prefill_small_zipf", 2),
               ("prefill_ksplit4_ragged", 2), ("n10k_prefill", 2), ("k_equals_E", 2)]


@pytest.mark.parametrize("name, path", TABLE_CASES)
def test_forward_routing_tables_bit_exact(m, name, path):
    """The dispatch arrays the forward itself used (decode: no padding, tile_m 1;
    prefill: segments padded to 256 rows), compared element by element with the
    oracle's dispatch of the same expert choice, and the choice with the oracle's."""
    wl = SMALL[name]
    inp = _inputs(wl, 11)
    t = synth.to_torch(inp)
    ws = m.alloc_workspace(H.shape_of(m, wl, path))
    ws.fill_(0x7B)
    L, r = _forward_tables(m, wl, t, path, ws)
    assert L["path"] == path
    T0 = wl.T - L["tokens"]
    dec = oracle.decode_workload_inputs(inp, wl)
    l, p, _, _ = oracle.route(dec["x"][T0:], dec["Wr"], dec["b"], wl.k)
    H.check_ids(r["topk_ids"], l, wl.k)
    w_ref = oracle.renormalize(p, r["topk_ids"].astype(np.int64))
    assert np.allclose(r["topk_w"], w_ref, rtol=2e-6, atol=1e-7)
    d = oracle.dispatch(r["topk_ids"].astype(np.int64), wl.E, L["tile_m"])
    assert L["capacity"] == d["capacity"]
    keys = ("counts", "offsets", "sorted_ids", "inv") + (("tile_expert",) if L["n_tiles"] else ())
    for key in keys:
        assert np.array_equal(r[key], d[key]), key
    act = r["active"]
    assert act[0] == len(d["active"]) and np.array_equal(act[1:1 + act[0]], d["active"])


@pytest.mark.parametrize("T, E, k", [(1, 256, 8), (3, 64, 8), (4, 8, 2), (40, 16, 6), (5, 256, 70), (2, 100, 12)])
def test_equal_logits_pick_lowest_indices(m, T, E, k):
    """All logits equal (zero router weights, no bias): every token takes experts
    0..k-1 in index order with weight 1/k, on each selection strategy."""
    wl = W(f"ties_{T}_{E}_{k}", T=T, H=64, E=E, k=k, I=32)
    inp = _inputs(wl, 7)
    inp["router_w"] = np.zeros_like(inp["router_w"])
    r = H.run_route(m, wl, synth.to_torch(inp))
    assert np.array_equal(r["topk_ids"], np.tile(np.arange(k), (T, 1)))
    assert np.allclose(r["topk_w"], 1.0 / k, rtol=1e-6)
    d = oracle.dispatch(r["topk_ids"].astype(np.int64), E, r["tile_m"])
    for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv"):
        assert np.array_equal(r[key], d[key]), key


@pytest.mark.parametrize("name,path", [("deepseek_small_t40", 1), ("deepseek_small_t40", 3),
                                       ("prefill_ksplit4_shared", 2), ("prefill_small_zipf", 2)])
def test_forward_is_deterministic(m, name, path):
    """Repeated calls give the same bits: no path adds with float atomics
    (the prefill combine sums each token's partial rows in a fixed order)."""
    import torch
    wl = SMALL[name]
    t = synth.to_torch(_inputs(wl, 5))
    ws = m.alloc_workspace(H.shape_of(m, wl, path))
    a = H.run_forward(m, wl, t, path=path, ws=ws).clone()
    for _ in range(3):
        b = H.run_forward(m, wl, t, path=path, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_needs_no_initialisation(m):
    """A workspace filled with garbage serves calls of different shapes and
    paths in a row: nothing in it has to be prepared or survives a call."""
    import torch
    big = SMALL["prefill_small_zipf"]
    ws = m.alloc_workspace(H.shape_of(m, big))
    ws.fill_(0xA5)
    for name in ("deepseek_small_t8", "prefill_small_zipf", "deepseek_small_t40", "qwen_small_q4_t5",
                 "deepseek_small_t8"):
        wl = SMALL[name]
        need = m.moe_workspace_size(H.shape_of(m, wl))
        assert need <= ws.numel() or name == "qwen_small_q4_t5"
        w = ws if need <= ws.numel() else m.alloc_workspace(H.shape_of(m, wl)).fill_(0x5A)
        inp = _inputs(wl, 6)
        t = synth.to_torch(inp)
        out = H.run_forward(m, wl, t, ws=w)
        torch.cuda.synchronize()
        err = H.relerr(H.to_f64(out), H.oracle_layer(wl, inp)["out"])
        assert err <= H.tolerance(wl), (name, err)


# -------------------------------------------------------------- full size ----

FULL = ["mixtral_decode_t8", "qwen_a3b_decode_q4", "deepseek16b_decode_t8", "deepseek16b_decode_t64",
        "mixtral_prefill_t4096", "mixtral_decode_t8_fp8", "qwen_a3b_decode_q8"]


@pytest.fixture(scope="module")
def full_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            import torch
            torch.cuda.empty_cache()
            cache[name] = synth.make_inputs_torch(synth.WORKLOADS[name], seed=0)
        return cache[name]
    return get


@pytest.mark.parametrize("name", FULL)
def test_full_size_route(m, full_inputs, name):
    wl = synth.WORKLOADS[name]
    t = full_inputs(name)
    r = H.run_route(m, wl, t)
    x = H.to_f64(t["x"])
    l = oracle.router_logits(x, H.to_f64(t["router_w"]), None if t["router_b"] is None else H.to_f64(t["router_b"]))
    n_diff, n_ties = H.check_ids(r["topk_ids"], l, wl.k)
    print(f"{name}: near-tie tokens {n_ties}, differing {n_diff}", flush=True)
    d = oracle.dispatch(r["topk_ids"].astype(np.int64), wl.E, r["tile_m"])
    for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv"):
        assert np.array_equal(r[key], d[key]), key


def _stratified_tokens(wl, r, rng):
    """Tokens of a full-size call to check against the oracle: every token up to
    64 of them; beyond that, for each expert the tokens of the first and last
    rows of its segment in the 256-padded prefill order and of the rows on
    either side of each 128-row half-tile boundary inside it, plus a few at
    random."""
    if wl.T <= 64:
        return np.arange(wl.T)
    ids = r["topk_ids"].astype(np.int64)
    d = oracle.dispatch(ids, wl.E, 256)
    n = wl.T * wl.k
    pick = set()
    for e in range(wl.E):
        c = int(d["counts"][e])
        if c == 0:
            continue
        o = int(d["offsets"][e])
        rows = {0, c - 1}
        for b in range(128, c + 128, 128):        # half-tile boundaries inside the segment
            rows.update(q for q in (b - 1, b) if q < c)
        for q in rows:
            f = int(d["sorted_ids"][o + q])
            assert f < n
            pick.add(f // wl.k)
    pick.update(int(v) for v in rng.choice(wl.T, size=6, replace=False))
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", FULL)
def test_full_size_forward_sampled(m, full_inputs, name):
    import torch
    wl = synth.WORKLOADS[name]
    t = full_inputs(name)
    out = H.run_forward(m, wl, t)
    r = H.run_route(m, wl, t)
    torch.cuda.synchronize()
    got = H.to_f64(out)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(0)
    tokens = _stratified_tokens(wl, r, rng)
    ref, l, _ = H.oracle_tokens(wl, t, tokens)
    ids_gpu = r["topk_ids"][tokens]
    if (ids_gpu != oracle.select_topk(l, wl.k)).any():
        H.check_ids(ids_gpu, l, wl.k)
        ref, _, _ = H.oracle_tokens(wl, t, tokens, ids_gpu=ids_gpu.astype(np.int64))
    err = H.relerr(got[tokens], ref)
    print(f"{name}: {len(tokens)} sampled tokens relerr {err:.3e}", flush=True)
    assert err <= 1e-2, err


@pytest.mark.parametrize("name", [n for n in FULL if "decode" in n and _fused_ok(synth.WORKLOADS[n])])
def test_full_size_decode_paths_agree(m, full_inputs, name):
    """At the benchmarked sizes the single-launch and multi-launch decode agree
    up to the order of their fp32 sums (each is checked against the oracle on
    its own by the sampled test)."""
    import torch
    wl = synth.WORKLOADS[name]
    t = full_inputs(name)
    multi = H.run_forward(m, wl, t, path=1)
    fused = H.run_forward(m, wl, t, path=3)
    torch.cuda.synchronize()
    assert H.same_up_to_rounding(fused, multi)


@pytest.mark.parametrize("name, path", [("deepseek_small_t40", 1), ("qwen_small_q4_t5", 0),
                                        ("deepseek_small_t8", 3), ("prefill_small_zipf", 2),
                                        # eager: selection inside the logits launch; captured: its own launch
                                        ("e32_t40_passes", 1)])
def test_graph_replay_matches_eager(m, name, path):
    """The layer captured into a HIP graph: several replays, with eager work and
    synchronisations between them, each equal to the eager result.  (A captured
    single-launch decode records the multi-launch decode, whose bits are the
    same.)"""
    import torch
    wl = SMALL[name]
    t = synth.to_torch(_inputs(wl, 7))
    shape = H.shape_of(m, wl, path)
    ws = m.alloc_workspace(shape)
    eager = H.run_forward(m, wl, t, path=path, ws=ws).clone()
    out = torch.empty_like(eager)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        m.moe_forward(shape, t["x"], t["router_w"], t["router_b"], t["w_gate"], t["w_up"], t["w_down"],
                      t.get("ws_gate"), t.get("ws_up"), t.get("ws_down"), out, ws, stream=cap.cuda_stream)
    for r in range(4):
        out.fill_(float("nan"))
        H.run_forward(m, wl, t, path=path, ws=ws)          # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # every path is deterministic: bit-exact
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           eager.view(torch.int16) if eager.dtype == torch.bfloat16 else eager), r


@pytest.mark.parametrize("name", ["e32_t40_passes", "dn_w8_passes_t32"])
def test_selection_in_logits_launch_reports_a_wait_that_gives_up(m, name):
    """A decode pass of more than 16 tokens with shared experts selects inside
    the logits launch, in a work-group that waits for the logit work-groups'
    flags.  With the wait bound forced to 0 from the host the wait gives up at
    once: every kernel still exits, the routing tables stay well formed (the
    selection runs on whatever logits are there) and the status words report
    it; a normal call afterwards reports success and matches the oracle."""
    import os
    import torch
    wl = SMALL[name]
    shape = H.shape_of(m, wl, 1)
    assert m.moe_forward_tables(shape)["shared_in_router"] == 1
    t = synth.to_torch(_inputs(wl, 13))
    ws = m.alloc_workspace(shape)
    ws.fill_(0x3C)
    old = os.environ.get("MOE_FUSED_WAIT_ROUNDS")
    os.environ["MOE_FUSED_WAIT_ROUNDS"] = "0"
    try:
        H.run_forward(m, wl, t, path=1, ws=ws)
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["MOE_FUSED_WAIT_ROUNDS"]
        else:
            os.environ["MOE_FUSED_WAIT_ROUNDS"] = old
    assert not m.fused_status_ok(shape, ws)
    out = H.run_forward(m, wl, t, path=1, ws=ws)
    torch.cuda.synchronize()
    assert m.fused_status_ok(shape, ws)
    inp = _inputs(wl, 13)
    ref = H.oracle_layer(wl, inp)
    assert H.relerr(H.to_f64(out), ref["out"]) <= H.tolerance(wl)


@pytest.mark.parametrize("name", ["deepseek_small_t8", "qwen_small_q4_t1", "e32_t40_passes"])
def test_single_launch_decode_reports_a_wait_that_gives_up(m, name):
    """The single-launch decode with its wait bound forced to 0 from the host:
    every wait gives up at once, so every item that depends on another skips
    its body and every work-group still exits.  The output must be all NaN
    and the status words must report the failure; a normal call on the same
    workspace afterwards reports success and equals the multi-launch decode."""
    import os
    import torch
    wl = SMALL[name]
    t = synth.to_torch(_inputs(wl, 12))
    shape = H.shape_of(m, wl, 3)
    ws = m.alloc_workspace(shape)
    ws.fill_(0x3C)
    old = os.environ.get("MOE_FUSED_WAIT_ROUNDS")
    os.environ["MOE_FUSED_WAIT_ROUNDS"] = "0"
    try:
        out = H.run_forward(m, wl, t, path=3, ws=ws)
        torch.cuda.synchronize()
    finally:
        if old is None:
            del os.environ["MOE_FUSED_WAIT_ROUNDS"]
        else:
            os.environ["MOE_FUSED_WAIT_ROUNDS"] = old
    last = H.to_f64(out)[wl.T - m.moe_forward_tables(shape)["tokens"]:]
    assert np.isnan(last).all()
    assert not m.fused_status_ok(shape, ws)
    fused = H.run_forward(m, wl, t, path=3, ws=ws)
    multi = H.run_forward(m, wl, t, path=1)
    torch.cuda.synchronize()
    assert m.fused_status_ok(shape, ws)
    assert H.same_up_to_rounding(fused, multi)
