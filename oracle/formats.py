"""Decoding of the stored input formats into exact float64 values.

bf16 and fp16 values convert to float64 exactly, and a Q4_0 weight d*(q-8)
(fp16 d, 4-bit q) is exact in float64, so the oracle always sees the very
values the GPU path reads.

Q4_0 ("Why MoE on RTX 5090 falls short: a bandwidth measurement",
news.malakhovai.ru, test-bench paragraph, names the Q4_0 quantisation of the
measured model; the block of 32 values with one fp16 scale d, 4-bit unsigned
codes q and value d*(q-8) is the workload's stated format).  Storage reading:
a stack [E, N, K] keeps all nibble bytes [E, N, K/2] first and then, from the
next 256-byte boundary, the fp16 scales [E, N, K/32].  In one block, value
j < 16 is the low nibble of byte j and value j + 16 the high nibble.

Q8_0 (named in the same test-bench paragraph among the quantisations of the
measured model, and as the stored format of the model run in "FATE: speeding
up MoE inference in llama.cpp with an expert cache and prefetching",
ai-manual.ru, section "How to use FATE: from build to first run").  Reading:
the Q4_0 block structure with signed 8-bit codes and no offset, value d*q;
storage as for Q4_0: all codes [E, N, K] (int8) first, then from the next
256-byte boundary the fp16 scales [E, N, K/32].

FP8 E4M3 (not on the pages: the 8-bit float that MI355X converts natively,
defined by the OCP 8-bit floating point specification).  A code is sign,
4 exponent bits with bias 7 and 3 mantissa bits; exponent 0 holds the
subnormals m/8 * 2^-6; S.1111.111 is NaN and there are no infinities, so the
largest value is 448.  Reading: one fp32 scale per output row (the row of
the weight matrix), value = scale * E4M3(code); storage: all codes [E, N, K]
first, then from the next 256-byte boundary the fp32 scales [E, N].
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 stored as uint16 bits -> float64 (exact): the bits are the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(bits_or_half: np.ndarray) -> np.ndarray:
    """IEEE binary16 (as float16 or as uint16 bits) -> float64 (exact)."""
    a = np.ascontiguousarray(bits_or_half)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def q4_0_decode(buf: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Q4_0 SoA stack [E, N, K] -> float64 values d*(q-8), shape [E, N, K]."""
    if K % 32:
        raise ValueError("Q4_0 needs K % 32 == 0")
    buf = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1)
    n_nib = E * N * K // 2
    nib = buf[:n_nib].reshape(E, N, K // 32, 16)
    low = (nib & 0x0F).astype(np.int64)          # values 0..15 of each block
    high = (nib >> 4).astype(np.int64)           # values 16..31 of each block
    q = np.concatenate([low, high], axis=-1)     # [E, N, K/32, 32]
    off = (n_nib + 255) // 256 * 256
    n_sc = E * N * (K // 32)
    d = buf[off:off + 2 * n_sc].view(np.float16).astype(np.float64).reshape(E, N, K // 32, 1)
    return (d * (q - 8)).reshape(E, N, K)


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64, exactly, from the field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    out = sign * mag
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, out)


def q8_0_matrix(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """One Q8_0 matrix: int8 codes [N, K] and fp16 scales [N, K/32] -> float64 d*q [N, K]."""
    q = np.asarray(codes).view(np.int8).astype(np.float64)
    N, K = q.shape
    return (f16_to_f64(np.asarray(d)).reshape(N, K // 32, 1) * q.reshape(N, K // 32, 32)).reshape(N, K)


def fp8_e4m3_matrix(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """One fp8 matrix: E4M3 codes [N, K] and fp32 row scales [N] -> float64 [N, K]."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return s.reshape(-1, 1) * fp8_e4m3_to_f64(codes)


def _scale_offset(n_codes: int) -> int:
    return (n_codes + 255) // 256 * 256


def q8_0_decode(buf: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Q8_0 SoA stack [E, N, K] -> float64 d*q, shape [E, N, K]."""
    if K % 32:
        raise ValueError("Q8_0 needs K % 32 == 0")
    buf = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1)
    n = E * N * K
    off = _scale_offset(n)
    d = buf[off:off + 2 * E * N * (K // 32)].view(np.uint16).reshape(E, N, K // 32)
    codes = buf[:n].reshape(E, N, K)
    return np.stack([q8_0_matrix(codes[e], d[e]) for e in range(E)])


def fp8_e4m3_decode(buf: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """fp8 E4M3 stack [E, N, K] with fp32 row scales -> float64 [E, N, K]."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1)
    n = E * N * K
    off = _scale_offset(n)
    s = buf[off:off + 4 * E * N].view(np.float32).reshape(E, N)
    codes = buf[:n].reshape(E, N, K)
    return np.stack([fp8_e4m3_matrix(codes[e], s[e]) for e in range(E)])


def weights_to_f64(a, dtype: str, shape) -> np.ndarray:
    """Stored weights of the given dtype ('f32' | 'bf16' | 'q4_0' | 'q8_0' | 'fp8_e4m3') -> float64 [*shape]."""
    if a is None:
        return None
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64).reshape(shape)
    if dtype == "bf16":
        return bf16_to_f64(a).reshape(shape)
    if dtype == "q4_0":
        return q4_0_decode(a, *shape)
    if dtype == "q8_0":
        return q8_0_decode(a, *shape)
    if dtype == "fp8_e4m3":
        return fp8_e4m3_decode(a, *shape)
    raise ValueError(dtype)


def decode_inputs(inp: dict, T, H, E, I, S, Is, x_dtype, w_dtype, r_dtype) -> dict:
    """Decode one layer call's stored inputs (as produced by the input generator)
    into float64 arrays: x [T,H], Wr [E,H], b [E] or None, Wg/Wu [E,I,H], Wd [E,H,I],
    shared = None or (Wsg [S,Is,H], Wsu [S,Is,H], Wsd [S,H,Is])."""
    x = weights_to_f64(inp["x"], x_dtype, (T, H))
    Wr = weights_to_f64(inp["router_w"], r_dtype, (E, H))
    b = None if inp.get("router_b") is None else np.asarray(inp["router_b"], np.float32).astype(np.float64)
    Wg = weights_to_f64(inp["w_gate"], w_dtype, (E, I, H))
    Wu = weights_to_f64(inp["w_up"], w_dtype, (E, I, H))
    Wd = weights_to_f64(inp["w_down"], w_dtype, (E, H, I))
    shared = None
    if S > 0:
        shared = (weights_to_f64(inp["ws_gate"], w_dtype, (S, Is, H)),
                  weights_to_f64(inp["ws_up"], w_dtype, (S, Is, H)),
                  weights_to_f64(inp["ws_down"], w_dtype, (S, H, Is)))
    return dict(x=x, Wr=Wr, b=b, Wg=Wg, Wu=Wu, Wd=Wd, shared=shared)


def decode_workload_inputs(inp: dict, wl) -> dict:
    """``decode_inputs`` with the sizes and dtypes read from a workload description."""
    return decode_inputs(inp, wl.T, wl.H, wl.E, wl.I, wl.S, wl.Is, wl.x_dtype, wl.w_dtype, wl.r_dtype)


def q4_0_decode_matrix(buf: np.ndarray, n_mat: int, N: int, K: int, e: int) -> np.ndarray:
    """Matrix e of a Q4_0 SoA stack [n_mat, N, K] -> float64 [N, K] (same reading as q4_0_decode)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8).reshape(-1)
    per_nib = N * K // 2
    nib = buf[e * per_nib:(e + 1) * per_nib].reshape(N, K // 32, 16)
    q = np.concatenate([(nib & 0x0F).astype(np.int64), (nib >> 4).astype(np.int64)], axis=-1)
    off = (n_mat * per_nib + 255) // 256 * 256
    per_sc = N * (K // 32)
    d = buf[off + 2 * e * per_sc: off + 2 * (e + 1) * per_sc].view(np.float16).astype(np.float64)
    return (d.reshape(N, K // 32, 1) * (q - 8)).reshape(N, K)
