"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The source pages print no worked numerical example, so the pins are closed
forms worked out by hand, hand-written bit patterns of the stored formats,
special cases, and a brute-force loop implementation on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import loops
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- formats ----

def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x0000, 0x8000, 0x7F80, 0x3F81, 0x4120],
                    dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 0.0, -0.0, math.inf, 1.0 + 2.0 ** -7, 10.0]
    got = oracle.bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w


def test_f16_bit_patterns():
    bits = np.array([0x3C00, 0x0001, 0xC000, 0x7BFF], dtype=np.uint16)
    got = oracle.f16_to_f64(bits)
    assert list(got) == [1.0, 2.0 ** -24, -2.0, 65504.0]


def test_bf16_rounding_ties_to_even():
    a = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e38], dtype=np.float32)
    got = synth.f32_to_bf16_bits(a)
    # 1+2^-8 is halfway between 0x3F80 and 0x3F81 -> even 0x3F80;
    # 1+3*2^-8 is halfway between 0x3F81 and 0x3F82 -> even 0x3F82.
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]


def _hand_q4_block(d_bits, codes):
    """One 32-value block written byte by byte: byte j = q_j | q_{j+16} << 4."""
    nib = bytes((codes[j] | (codes[j + 16] << 4)) for j in range(16))
    return nib, d_bits.to_bytes(2, "little")


def test_q4_0_hand_block():
    codes = list(range(16)) + list(range(15, -1, -1))
    nib, d = _hand_q4_block(0x3C00, codes)                # d = 1.0
    buf = np.zeros(256 + 2, dtype=np.uint8)
    buf[:16] = np.frombuffer(nib, dtype=np.uint8)
    buf[256:258] = np.frombuffer(d, dtype=np.uint8)       # scales start at the next 256-byte boundary
    w = oracle.q4_0_decode(buf, 1, 1, 32)[0, 0]
    assert list(w[:16]) == [float(v) for v in range(-8, 8)]
    assert list(w[16:]) == [float(v) for v in range(7, -9, -1)]


def test_q4_0_two_rows_two_blocks_scale_indexing():
    # rows r=0,1; blocks b=0,1; scale of (r, b) = 2^(r*2+b-1); all codes 9 -> q-8 = 1
    E, N, K = 1, 2, 64
    nib = np.full(E * N * K // 2, 0x99, dtype=np.uint8)
    scales = np.array([0.5, 1.0, 2.0, 4.0], dtype=np.float16)
    buf = np.zeros(256 + 8, dtype=np.uint8)
    buf[:nib.size] = nib
    buf[256:] = scales.view(np.uint8)
    w = oracle.q4_0_decode(buf, E, N, K)[0]
    assert np.all(w[0, :32] == 0.5) and np.all(w[0, 32:] == 1.0)
    assert np.all(w[1, :32] == 2.0) and np.all(w[1, 32:] == 4.0)


def test_generator_q4_layout_matches_hand_bytes():
    codes = np.array(list(range(16)) + list(range(15, -1, -1)), dtype=np.uint8).reshape(1, 1, 32)
    buf = synth.q4_0_pack(codes, np.array([[[1.0]]], dtype=np.float16))
    nib, d = _hand_q4_block(0x3C00, list(codes.reshape(-1)))
    assert bytes(buf[:16]) == nib
    assert bytes(buf[256:258]) == d
    assert buf.size == synth.q4_0_nbytes(1, 1, 32) == 258


def test_q4_special_values():
    E, N, K = 2, 3, 64
    q = np.full((E, N, K), 8, dtype=np.uint8)
    d = np.full((E, N, K // 32), 0.75, dtype=np.float16)
    assert np.all(oracle.q4_0_decode(synth.q4_0_pack(q, d), E, N, K) == 0.0)    # q == 8 -> 0
    q2 = np.random.default_rng(1).integers(0, 16, size=(E, N, K), dtype=np.uint8)
    assert np.all(oracle.q4_0_decode(synth.q4_0_pack(q2, np.zeros_like(d)), E, N, K) == 0.0)  # d == 0


# ------------------------------------------------------------ closed forms ---

LN3 = math.log(3.0)


def test_router_closed_form():
    # logits [ln 3, 0] -> p = [3/4, 1/4]
    x = np.array([[1.0, 0.0]])
    Wr = np.array([[LN3, 0.0], [0.0, 5.0]])
    l, p, ids, w = oracle.route(x, Wr, None, 1)
    assert l.tolist() == [[LN3, 0.0]]
    assert np.allclose(p, [[0.75, 0.25]], rtol=0, atol=1e-15)
    assert ids.tolist() == [[0]] and w.tolist() == [[1.0]]
    _, _, ids2, w2 = oracle.route(x, Wr, None, 2)
    assert ids2.tolist() == [[0, 1]]
    assert np.allclose(w2, [[0.75, 0.25]], rtol=0, atol=1e-15)


def test_router_bias_moves_selection():
    x = np.array([[1.0, 0.0]])
    Wr = np.array([[LN3, 0.0], [0.0, 5.0]])
    b = np.array([0.0, 2.0])          # logits [ln3, 2] -> expert 1 wins
    _, p, ids, w = oracle.route(x, Wr, b, 1)
    assert ids.tolist() == [[1]]
    assert np.allclose(p[0], np.array([3.0, math.e ** 2]) / (3.0 + math.e ** 2), rtol=1e-15)


def test_all_ties_pick_lowest_indices():
    T, H, E = 3, 8, 6
    x = np.random.default_rng(0).standard_normal((T, H))
    for k in (1, 3, 6):
        _, _, ids, w = oracle.route(x, np.zeros((E, H)), None, k)
        assert ids.tolist() == [list(range(k))] * T
        assert np.allclose(w, 1.0 / k, rtol=1e-15, atol=0)


def test_silu_closed_forms():
    z = np.array([0.0, LN3, -LN3, 40.0, -800.0])
    got = oracle.silu(z)
    # silu(ln3) = ln3 * 3/4; silu(-ln3) = -ln3 * 1/4; silu(40) ~ 40; silu(-800) -> -0
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * LN3) < 1e-15
    assert abs(got[2] + 0.25 * LN3) < 1e-15
    assert abs(got[3] - 40.0) < 1e-12
    assert got[4] == 0.0


def test_swiglu_closed_form():
    # g = ln3, u = 2 -> a = silu(ln3) * 2 = 1.5 ln3 ; y = Wd a = [1.5 ln3, -1.5 ln3, 3 ln3]
    x = np.array([[1.0, 0.0, 0.0]])
    Wg = np.array([[LN3, 0.0, 7.0]])
    Wu = np.array([[2.0, 0.0, -1.0]])
    Wd = np.array([[1.0], [-1.0], [2.0]])
    y = oracle.swiglu_ffn(x, Wg, Wu, Wd)
    assert np.allclose(y, [[1.5 * LN3, -1.5 * LN3, 3.0 * LN3]], rtol=1e-15, atol=0)


def test_layer_closed_form_with_shared_expert():
    # Router logits [ln3, 0]: top-2 weights [3/4, 1/4]; expert 0 gives y0 = [1.5 ln3, -1.5 ln3, 3 ln3];
    # expert 1 has zero down weights; the shared expert has g = ln3, u = 4 -> a = 3 ln3 and
    # down [[1],[0],[0]] -> [3 ln3, 0, 0], added with weight 1.
    x = np.array([[1.0, 0.0, 0.0]])
    Wr = np.array([[LN3, 0.0, 0.0], [0.0, 0.0, 0.0]])
    Wg = np.array([[[LN3, 0.0, 0.0]], [[1.0, 0.0, 0.0]]])
    Wu = np.array([[[2.0, 0.0, 0.0]], [[1.0, 0.0, 0.0]]])
    Wd = np.array([[[1.0], [-1.0], [2.0]], [[0.0], [0.0], [0.0]]])
    shared = (np.array([[[LN3, 0.0, 0.0]]]), np.array([[[4.0, 0.0, 0.0]]]),
              np.array([[[1.0], [0.0], [0.0]]]))
    r = oracle.moe_forward(x, Wr, None, Wg, Wu, Wd, 2, shared)
    want = np.array([[0.75 * 1.5 * LN3 + 3.0 * LN3, -0.75 * 1.5 * LN3, 0.75 * 3.0 * LN3]])
    assert np.allclose(r["out"], want, rtol=1e-15, atol=1e-15)
    out_l, ids_l, w_l = loops.moe_forward(x.tolist(), Wr.tolist(), None, Wg.tolist(), Wu.tolist(),
                                          Wd.tolist(), 2, tuple(s.tolist() for s in shared))
    assert np.allclose(out_l, want, rtol=1e-15, atol=1e-15)


def test_golden_hand_example(root):
    """tests/golden/hand_layer.txt: the closed-form layer above, values derived by hand."""
    path = f"{root}/tests/golden/hand_layer.txt"
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = [float(s) for s in v.split()]
    x = np.array([[1.0, 0.0, 0.0]])
    Wr = np.array([[LN3, 0.0, 0.0], [0.0, 0.0, 0.0]])
    Wg = np.array([[[LN3, 0.0, 0.0]], [[1.0, 0.0, 0.0]]])
    Wu = np.array([[[2.0, 0.0, 0.0]], [[1.0, 0.0, 0.0]]])
    Wd = np.array([[[1.0], [-1.0], [2.0]], [[0.0], [0.0], [0.0]]])
    r = oracle.moe_forward(x, Wr, None, Wg, Wu, Wd, 2, None)
    assert np.allclose(r["p"][0], vals["p"], rtol=1e-12)
    assert np.allclose(r["w"][0], vals["w"], rtol=1e-12)
    assert np.allclose(r["out"][0], vals["out_no_shared"], rtol=1e-12)


# --------------------------------------------------------------- dispatch ----

def test_dispatch_hand_example_full_segments():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    d = oracle.dispatch(ids, E=3, M=2)
    assert d["counts"].tolist() == [2, 2, 2]
    assert d["offsets"].tolist() == [0, 2, 4, 6]
    assert d["sorted_ids"].tolist() == [1, 2, 3, 5, 0, 4, 6, 6, 6, 6]
    assert d["tile_expert"].tolist() == [0, 1, 2, -1, -1]
    assert d["inv"].tolist() == [4, 0, 1, 2, 5, 3]
    assert d["active"].tolist() == [0, 1, 2]


def test_dispatch_hand_example_padding_and_empty_expert():
    ids = np.array([[3, 1], [1, 3], [1, 0]])
    d = oracle.dispatch(ids, E=4, M=4)
    assert d["counts"].tolist() == [1, 3, 0, 2]
    assert d["offsets"].tolist() == [0, 4, 8, 8, 12]
    s = 6
    assert d["sorted_ids"].tolist() == [5, s, s, s, 1, 2, 4, s, 0, 3, s, s] + [s] * 8
    assert d["tile_expert"].tolist() == [0, 1, 3, -1, -1]
    assert d["active"].tolist() == [0, 1, 3]
    assert d["inv"].tolist() == [8, 4, 5, 9, 6, 0]


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E = int(rng.integers(1, 40)), int(rng.integers(1, 12))
    k = int(rng.integers(1, E + 1))
    M = int(rng.choice([1, 2, 4, 16]))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    a = oracle.dispatch(ids, E, M)
    b = loops.dispatch(ids.tolist(), E, M)
    for key in ("counts", "offsets", "sorted_ids", "tile_expert", "inv", "active"):
        assert list(a[key]) == list(b[key]), key
    assert a["capacity"] == b["capacity"] == oracle.padded_rows(T, k, E, M)
    # invariants
    n = T * k
    assert a["counts"].sum() == n
    assert np.all(np.diff(a["offsets"]) % M == 0)
    real = a["sorted_ids"][a["sorted_ids"] != n]
    assert sorted(real.tolist()) == list(range(n))
    assert np.all(a["sorted_ids"][a["inv"]] == np.arange(n))


# ------------------------------------------------------------ brute force ----

def _tiny(seed, T, H, E, k, I, S=0, Is=0, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((E, H)) * 0.5
    b = rng.standard_normal(E) if bias else None
    Wg = rng.standard_normal((E, I, H)) * 0.3
    Wu = rng.standard_normal((E, I, H)) * 0.3
    Wd = rng.standard_normal((E, H, I)) * 0.3
    shared = None
    if S:
        shared = (rng.standard_normal((S, Is, H)) * 0.3, rng.standard_normal((S, Is, H)) * 0.3,
                  rng.standard_normal((S, H, Is)) * 0.3)
    return x, Wr, b, Wg, Wu, Wd, shared


@pytest.mark.parametrize("case", [
    dict(seed=0, T=3, H=5, E=4, k=2, I=6),
    dict(seed=1, T=4, H=8, E=6, k=3, I=4, bias=True),
    dict(seed=2, T=2, H=7, E=3, k=3, I=5, S=1, Is=3),
    dict(seed=3, T=5, H=4, E=5, k=1, I=2, S=2, Is=4, bias=True),
    dict(seed=4, T=1, H=6, E=1, k=1, I=3),
])
def test_vectorised_matches_brute_force(case):
    x, Wr, b, Wg, Wu, Wd, shared = _tiny(**case)
    r = oracle.moe_forward(x, Wr, b, Wg, Wu, Wd, case["k"], shared)
    sh = None if shared is None else tuple(s.tolist() for s in shared)
    out, ids, w = loops.moe_forward(x.tolist(), Wr.tolist(), b, Wg.tolist(), Wu.tolist(),
                                    Wd.tolist(), case["k"], sh)
    assert r["ids"].tolist() == ids
    assert np.allclose(r["w"], w, rtol=1e-13, atol=0)
    assert np.allclose(r["out"], out, rtol=1e-12, atol=1e-13)


def test_loop_router_ties_to_lower_index():
    x = [[1.0, 2.0]]
    Wr = [[1.0, 0.0], [0.5, 0.25], [1.0, 0.0], [0.0, 0.5]]   # logits 1, 1, 1, 1
    _, _, ids, w = loops.route_one(x[0], Wr, None, 3)
    assert ids == [0, 1, 2] and all(abs(v - 1 / 3) < 1e-15 for v in w)
    got = oracle.select_topk(np.array([[1.0, 1.0, 1.0, 1.0]]), 3)
    assert got.tolist() == [[0, 1, 2]]


def test_near_tie_flagging():
    l = np.array([[1.0, 0.99995, -3.0],    # gap 5e-5 between 1st and 2nd -> flagged for k = 1, 2
                  [1.0, 0.5, 0.49999],     # gap 1e-5 between 2nd and 3rd -> flagged for k = 2, not k = 1
                  [2.0, 1.0, 0.0]])
    assert oracle.near_ties(l, 1).tolist() == [True, False, False]
    assert oracle.near_ties(l, 2).tolist() == [True, True, False]
    assert oracle.near_ties(l, 3).tolist() == [True, True, False]


def test_q4_0_single_matrix_decode_matches_stack_decode():
    rng = np.random.default_rng(3)
    E, N, K = 3, 5, 96
    q = rng.integers(0, 16, size=(E, N, K), dtype=np.uint8)
    d = rng.random((E, N, K // 32)).astype(np.float16)
    buf = synth.q4_0_pack(q, d)
    full = oracle.q4_0_decode(buf, E, N, K)
    for e in range(E):
        assert np.array_equal(oracle.q4_0_decode_matrix(buf, E, N, K, e), full[e])
    # and both equal d * (q - 8) computed from the unpacked draws
    assert np.array_equal(full, d.astype(np.float64).repeat(32, axis=-1) * (q.astype(np.float64) - 8))


# ------------------------------------------------------------ Q8_0 / FP8 ----

# E4M3 codes worked out by hand from the OCP 8-bit floating point definition
# (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 subnormal).
E4M3_HAND = [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x30, 0.5), (0x3C, 1.5), (0x40, 2.0), (0x78, 256.0),
    (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x0F, 1.875 * 2.0 ** -6), (0x81, -(2.0 ** -9)),
]


def test_fp8_e4m3_hand_values():
    codes = np.array([c for c, _ in E4M3_HAND], dtype=np.uint8)
    got = oracle.fp8_e4m3_to_f64(codes)
    assert got.tolist() == [v for _, v in E4M3_HAND]
    assert np.signbit(oracle.fp8_e4m3_to_f64(np.array([0x80], np.uint8)))[0]      # -0
    assert np.isnan(oracle.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_fp8_e4m3_all_codes_match_library_decoder():
    """Every one of the 256 codes against PyTorch's own float8_e4m3fn decoding."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.fp8_e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], ours[ok])


def test_fp8_e4m3_positive_codes_increase():
    v = oracle.fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0) and v[-1] == 448.0


def test_q8_0_hand_block_and_scale_offset():
    """One row of two blocks: codes in the first 64 bytes, the two fp16 scales
    from byte 256 (the next 256-byte boundary)."""
    q = np.array(list(range(-16, 16)) + [127, -128] + [0] * 30, dtype=np.int8)
    buf = np.zeros(256 + 4, dtype=np.uint8)
    buf[:64] = q.view(np.uint8)
    buf[256:260] = np.array([0.5, -2.0], dtype=np.float16).view(np.uint8)
    w = oracle.q8_0_decode(buf, 1, 1, 64)[0, 0]
    assert w[:32].tolist() == [0.5 * v for v in range(-16, 16)]
    assert w[32] == -254.0 and w[33] == 256.0 and np.all(w[34:] == 0.0)


def test_fp8_stack_row_scales_and_matrix_index():
    """Two matrices of two rows: matrix e, row n scales by s[e, n]; the scales
    start at the 256-byte boundary after all codes."""
    E, N, K = 2, 2, 32
    codes = np.full((E, N, K), 0x38, dtype=np.uint8)      # 1.0
    codes[1, 0, 5] = 0xC0                                   # -2.0
    s = np.array([[1.0, 0.5], [3.0, -0.25]], dtype=np.float32)
    buf = np.zeros(256 + 16, dtype=np.uint8)
    buf[:E * N * K] = codes.reshape(-1)
    buf[256:272] = s.view(np.uint8).reshape(-1)
    w = oracle.fp8_e4m3_decode(buf, E, N, K)
    assert np.all(w[0, 0] == 1.0) and np.all(w[0, 1] == 0.5) and np.all(w[1, 1] == -0.25)
    assert w[1, 0, 5] == -6.0 and np.sum(w[1, 0] == 3.0) == K - 1


@pytest.mark.parametrize("dtype", ["q8_0", "fp8_e4m3"])
def test_generator_8bit_stacks_round_trip(dtype):
    """Stacks made by the input generator decode to within the format's own
    rounding of the normal values they were made from."""
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(3, 5, 64)).astype(np.float32)
    buf = synth.pack_weights(w, dtype)
    assert buf.size == synth.weight_nbytes(dtype, 3, 5, 64)
    dec = oracle.weights_to_f64(buf, dtype, (3, 5, 64))
    if dtype == "q8_0":      # |err| <= d/2 per block (plus fp16 rounding of d)
        d = np.abs(w.reshape(3, 5, 2, 32)).max(-1, keepdims=True) / 127
        assert np.all(np.abs(dec.reshape(3, 5, 2, 32) - w.reshape(3, 5, 2, 32)) <= 0.51 * d + 1e-7)
    else:                    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normals
        rel = np.abs(dec - w) / np.maximum(np.abs(w), 1e-30)
        s = np.abs(w).max(-1, keepdims=True) / 448
        assert np.all((rel <= 2.0 ** -4 + 1e-6) | (np.abs(w) < 2.0 ** -6 * s))
