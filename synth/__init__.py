"""Seeded synthetic inputs for the MoE layer forward.

This module only draws and lays out input data.  It holds none of the
layer's arithmetic: no routing, no softmax, no dequantisation, no FFN.  Both
the fp64 oracle and the HIP path consume the bits it produces, and each side
interprets them with its own code.

Workloads (sizes and distributions follow the model shapes that the source
pages discuss; weights are random because no trained checkpoints are used):

* ``tiny_f32``            T=4,    H=64,   E=4,   k=2, I=128,   no shared, fp32
* ``mixtral_decode_t8``   T=8,    H=4096, E=8,   k=2, I=14336, no shared, bf16
* ``qwen_a3b_decode_q4``  T=1,    H=2048, E=256, k=8, I=512, 1 shared (512),
                          Q4_0 experts, fp32 router, fp32 activations
* ``deepseek16b_decode_t8`` / ``_t64``  T=8 / 64, H=2048, E=64, k=6, I=1408,
                          2 shared (1408 each), bf16
* ``mixtral_prefill_t4096`` T=4096, H=4096, E=8, k=2, I=14336, bf16, router
                          bias ln(p_e) with p_e proportional to (e+1)^-1.2

Generation recipe (numpy ``default_rng(seed)``, PCG64), in this order:
x ~ N(0,1); router weights ~ N(0, 0.02^2); then for each routed expert e:
gate, up, down; then for each shared expert: gate, up, down.  Normal draws are
float32, scaled by the std in float32, then rounded to bf16 with
round-to-nearest-even when the dtype is bf16.  A Q4_0 matrix draws its 4-bit
codes q ~ U{0..15} first, then its scales d = fp16(|N(0, 0.002^2)|).

Q4_0 storage ("SoA"): a stack [E, N, K] with K % 32 == 0 is stored as all the
nibble bytes [E, N, K/2] first, then, from the next 256-byte boundary, all the
fp16 scales [E, N, K/32].  Inside one 32-value block, value j < 16 lives in
the low nibble of byte j and value j + 16 in the high nibble of byte j.  The
value it stands for is d * (q - 8).

Q8_0 and fp8 E4M3 stacks are made from normal weights N(0, 0.02^2) drawn
like the bf16 ones (float32): Q8_0 takes per block of 32 along K the scale
d = fp16(max|w| / 127) and the codes q = clip(round(w / d), -127, 127); fp8
takes per row the fp32 scale s = max|w| / 448 and the codes E4M3(w / s)
(nearest, ties to even; torch's float8_e4m3fn conversion).  Storage: all codes
[E, N, K] (one byte each) first, then from the next 256-byte boundary the
scales (Q8_0: fp16 [E, N, K/32]; fp8: fp32 [E, N]).

Large workloads can also be drawn on the GPU with ``torch`` generators
(``make_inputs_torch``); they then have the same shapes and distributions but
not the same bits as the numpy recipe.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32, BF16, Q4_0, Q8_0, FP8 = "f32", "bf16", "q4_0", "q8_0", "fp8_e4m3"
Q4_BLOCK = 32
Q4_ALIGN = 256


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    S: int = 0          # shared experts
    Is: int = 0         # shared-expert intermediate size
    x_dtype: str = BF16
    w_dtype: str = BF16
    r_dtype: str = BF16
    zipf_s: Optional[float] = None   # router bias ln p_e, p_e ~ (e+1)^-s
    channel_budget: Optional[float] = None   # channel-sparse experts: share of channels kept
    w_std: float = 0.02
    q4_d_std: float = 0.002

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", T=4, H=64, E=4, k=2, I=128,
                 x_dtype=F32, w_dtype=F32, r_dtype=F32),
        Workload("mixtral_decode_t8", T=8, H=4096, E=8, k=2, I=14336),
        Workload("qwen_a3b_decode_q4", T=1, H=2048, E=256, k=8, I=512, S=1, Is=512,
                 x_dtype=F32, w_dtype=Q4_0, r_dtype=F32),
        Workload("deepseek16b_decode_t8", T=8, H=2048, E=64, k=6, I=1408, S=2, Is=1408),
        Workload("deepseek16b_decode_t64", T=64, H=2048, E=64, k=6, I=1408, S=2, Is=1408),
        Workload("mixtral_prefill_t4096", T=4096, H=4096, E=8, k=2, I=14336, zipf_s=1.2),
        # 8-bit weight variants of two decode shapes
        Workload("mixtral_decode_t8_fp8", T=8, H=4096, E=8, k=2, I=14336, w_dtype=FP8),
        Workload("qwen_a3b_decode_q8", T=1, H=2048, E=256, k=8, I=512, S=1, Is=512,
                 x_dtype=F32, w_dtype=Q8_0, r_dtype=F32),
        # batch one, dense, and with budgeted channel sparsity (17.8 % of each engaged expert's channels)
        Workload("mixtral_decode_t1", T=1, H=4096, E=8, k=2, I=14336),
        Workload("mixtral_decode_t1_sparse", T=1, H=4096, E=8, k=2, I=14336, channel_budget=0.178),
    ]
}


# ----------------------------------------------------------------------------
# bit-level helpers (data layout only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def q4_0_nbytes(E: int, N: int, K: int) -> int:
    """Byte size of a Q4_0 SoA stack [E, N, K]."""
    nib = E * N * K // 2
    return _align(nib, Q4_ALIGN) + E * N * (K // Q4_BLOCK) * 2


def q4_0_pack(q: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """Lay out codes q [E,N,K] (uint8 0..15) and scales d [E,N,K/32] (float16)."""
    E, N, K = q.shape
    assert K % Q4_BLOCK == 0 and d_f16.shape == (E, N, K // Q4_BLOCK)
    blocks = q.reshape(E, N, K // Q4_BLOCK, Q4_BLOCK).astype(np.uint8)
    lo, hi = blocks[..., :16], blocks[..., 16:]
    nib = (lo | (hi << np.uint8(4))).astype(np.uint8).reshape(-1)
    buf = np.zeros(q4_0_nbytes(E, N, K), dtype=np.uint8)
    buf[: nib.size] = nib
    off = _align(nib.size, Q4_ALIGN)
    buf[off:] = np.ascontiguousarray(d_f16, dtype=np.float16).reshape(-1).view(np.uint8)
    return buf


def weight_nbytes(dtype: str, E: int, N: int, K: int) -> int:
    """Bytes of one stored weight stack [E, N, K]."""
    if dtype == F32:
        return 4 * E * N * K
    if dtype == BF16:
        return 2 * E * N * K
    if dtype == Q4_0:
        return q4_0_nbytes(E, N, K)
    if dtype == Q8_0:
        return _align(E * N * K, Q4_ALIGN) + 2 * E * N * (K // Q4_BLOCK)
    if dtype == FP8:
        return _align(E * N * K, Q4_ALIGN) + 4 * E * N
    raise ValueError(dtype)


def pack_weights(w: np.ndarray, dtype: str) -> np.ndarray:
    """Quantise float32 weights [E, N, K] to a Q8_0 or fp8 E4M3 stack (uint8 buffer)."""
    import torch
    w = np.ascontiguousarray(w, dtype=np.float32)
    E, N, K = w.shape
    buf = np.zeros(weight_nbytes(dtype, E, N, K), dtype=np.uint8)
    off = _align(E * N * K, Q4_ALIGN)
    if dtype == Q8_0:
        blk = w.reshape(E, N, K // Q4_BLOCK, Q4_BLOCK)
        d = (np.abs(blk).max(-1) / np.float32(127)).astype(np.float16)
        dd = d.astype(np.float32)[..., None]
        q = np.where(dd > 0, np.rint(blk / np.where(dd > 0, dd, 1)), 0)
        q = np.clip(q, -127, 127).astype(np.int8)
        buf[:E * N * K] = q.reshape(-1).view(np.uint8)
        buf[off:] = d.reshape(-1).view(np.uint8)
    elif dtype == FP8:
        sc = (np.abs(w).max(-1) / np.float32(448)).astype(np.float32)
        v = w / np.where(sc > 0, sc, 1)[..., None]
        codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        buf[:E * N * K] = codes.reshape(-1)
        buf[off:] = sc.reshape(-1).view(np.uint8)
    else:
        raise ValueError(dtype)
    return buf


def channel_count(w: Workload) -> int:
    """Channels kept per (token, engaged expert) for a channel-sparse workload."""
    return max(1, min(w.I, int(round(w.channel_budget * w.I))))


def channel_scores(w: Workload, seed: int) -> np.ndarray:
    """Per-token channel scores [T, E, I] (float32, N(0, 1)), from their own
    stream so that the other inputs of the same seed do not change.  They stand
    in for a selector's scores (the selector itself is not modelled)."""
    rng = np.random.default_rng([seed, 0x5C0E])
    return rng.standard_normal(size=(w.T, w.E, w.I), dtype=np.float32)


def down_transposed(a: np.ndarray, n: int, H: int, inter: int) -> np.ndarray:
    """A dense down stack [n, H, inter] (float32 or bf16 bits) laid out as
    [n, inter, H], so that one intermediate channel is one contiguous row."""
    return np.ascontiguousarray(np.asarray(a).reshape(n, H, inter).transpose(0, 2, 1))


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Router bias b_e = ln p_e with p_e proportional to (e+1)^-s (normalised)."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def _align(n: int, a: int) -> int:
    return (n + a - 1) // a * a


# ----------------------------------------------------------------------------
# numpy generator (bit-identical inputs for both sides)
# ----------------------------------------------------------------------------

def _normal(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == F32:
        return a
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def _q4_matrix(rng, E, N, K, d_std):
    q = rng.integers(0, 16, size=(E, N, K), dtype=np.uint8)
    d = np.abs(rng.standard_normal(size=(E, N, K // Q4_BLOCK), dtype=np.float32))
    d = (d * np.float32(d_std)).astype(np.float16)
    return q4_0_pack(q, d)


def _expert_stack(rng, w: Workload, n: int, inter: int):
    """gate [n, inter, H], up [n, inter, H], down [n, H, inter]; drawn expert by expert."""
    H = w.H
    if w.w_dtype in (Q8_0, FP8):
        g = np.empty((n, inter, H), dtype=np.float32)
        u = np.empty((n, inter, H), dtype=np.float32)
        d = np.empty((n, H, inter), dtype=np.float32)
        for e in range(n):
            g[e] = _normal(rng, (inter, H), w.w_std, F32)
            u[e] = _normal(rng, (inter, H), w.w_std, F32)
            d[e] = _normal(rng, (H, inter), w.w_std, F32)
        return pack_weights(g, w.w_dtype), pack_weights(u, w.w_dtype), pack_weights(d, w.w_dtype)
    if w.w_dtype == Q4_0:
        gs, us, ds = [], [], []
        for _ in range(n):
            gs.append((rng.integers(0, 16, size=(inter, H), dtype=np.uint8),
                       _q4_scales(rng, inter, H, w.q4_d_std)))
            us.append((rng.integers(0, 16, size=(inter, H), dtype=np.uint8),
                       _q4_scales(rng, inter, H, w.q4_d_std)))
            ds.append((rng.integers(0, 16, size=(H, inter), dtype=np.uint8),
                       _q4_scales(rng, H, inter, w.q4_d_std)))
        pack = lambda lst: q4_0_pack(np.stack([a for a, _ in lst]), np.stack([b for _, b in lst]))
        return pack(gs), pack(us), pack(ds)
    dt = np.float32 if w.w_dtype == F32 else np.uint16
    g = np.empty((n, inter, H), dtype=dt)
    u = np.empty((n, inter, H), dtype=dt)
    d = np.empty((n, H, inter), dtype=dt)
    for e in range(n):
        g[e] = _normal(rng, (inter, H), w.w_std, w.w_dtype)
        u[e] = _normal(rng, (inter, H), w.w_std, w.w_dtype)
        d[e] = _normal(rng, (H, inter), w.w_std, w.w_dtype)
    return g, u, d


def _q4_scales(rng, N, K, d_std):
    d = np.abs(rng.standard_normal(size=(N, K // Q4_BLOCK), dtype=np.float32))
    return (d * np.float32(d_std)).astype(np.float16)


def make_inputs(w: Workload, seed: int) -> dict:
    """Draw every input of one layer call.

    Returns a dict of numpy arrays holding stored bits: float32 arrays for
    fp32 data, uint16 arrays of bf16 bits for bf16 data, uint8 SoA buffers for
    Q4_0 stacks.  Keys: x, router_w, router_b (None or float32 [E]), w_gate,
    w_up, w_down, ws_gate, ws_up, ws_down (None when S == 0).
    """
    rng = np.random.default_rng(seed)
    x = _normal(rng, (w.T, w.H), 1.0, w.x_dtype)
    wr = _normal(rng, (w.E, w.H), w.w_std, w.r_dtype)
    b = zipf_bias(w.E, w.zipf_s) if w.zipf_s is not None else None
    g, u, d = _expert_stack(rng, w, w.E, w.I)
    if w.S > 0:
        sg, su, sd = _expert_stack(rng, w, w.S, w.Is)
    else:
        sg = su = sd = None
    return dict(x=x, router_w=wr, router_b=b, w_gate=g, w_up=u, w_down=d,
                ws_gate=sg, ws_up=su, ws_down=sd)


# ----------------------------------------------------------------------------
# torch generator on the GPU (same shapes and distributions, other bits)
# ----------------------------------------------------------------------------

def make_inputs_torch(w: Workload, seed: int, device="cuda", copies: int = 1) -> dict:
    """Draw one layer call's inputs with torch on ``device``.

    ``copies`` > 1 draws that many independent weight sets (a list per key) so
    that a timing loop can rotate through more bytes than the caches hold.
    Values are returned as torch tensors: float32, bfloat16, or uint8 (Q4_0).
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(shape, std, dtype):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        if dtype == F32:
            return t
        return t.to(torch.bfloat16)

    def q4(E, N, K):
        q = torch.randint(0, 16, (E, N, K), generator=gen, device=device, dtype=torch.uint8)
        d = torch.randn((E, N, K // Q4_BLOCK), generator=gen, device=device).abs_().mul_(w.q4_d_std)
        d = d.to(torch.float16)
        blocks = q.view(E, N, K // Q4_BLOCK, Q4_BLOCK)
        nib = (blocks[..., :16] | (blocks[..., 16:] << 4)).reshape(-1)
        buf = torch.zeros(q4_0_nbytes(E, N, K), dtype=torch.uint8, device=device)
        buf[: nib.numel()] = nib
        off = _align(nib.numel(), Q4_ALIGN)
        buf[off:] = d.reshape(-1).view(torch.uint8)
        return buf

    def q8_or_fp8(E, N, K):
        t = torch.randn((E, N, K), generator=gen, device=device, dtype=torch.float32).mul_(w.w_std)
        buf = torch.zeros(weight_nbytes(w.w_dtype, E, N, K), dtype=torch.uint8, device=device)
        off = _align(E * N * K, Q4_ALIGN)
        if w.w_dtype == Q8_0:
            blk = t.view(E, N, K // Q4_BLOCK, Q4_BLOCK)
            d = (blk.abs().amax(-1) / 127).to(torch.float16)
            dd = d.float().unsqueeze(-1)
            q = torch.where(dd > 0, torch.round(blk / torch.where(dd > 0, dd, torch.ones_like(dd))),
                            torch.zeros_like(blk)).clamp_(-127, 127).to(torch.int8)
            buf[: E * N * K] = q.reshape(-1).view(torch.uint8)
            buf[off:] = d.reshape(-1).view(torch.uint8)
        else:
            sc = t.abs().amax(-1) / 448
            v = t / torch.where(sc > 0, sc, torch.ones_like(sc)).unsqueeze(-1)
            buf[: E * N * K] = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(-1)
            buf[off:] = sc.reshape(-1).view(torch.uint8)
        return buf

    def stack(n, inter):
        if w.w_dtype == Q4_0:
            return q4(n, inter, w.H), q4(n, inter, w.H), q4(n, w.H, inter)
        if w.w_dtype in (Q8_0, FP8):
            return q8_or_fp8(n, inter, w.H), q8_or_fp8(n, inter, w.H), q8_or_fp8(n, w.H, inter)
        return (normal((n, inter, w.H), w.w_std, w.w_dtype),
                normal((n, inter, w.H), w.w_std, w.w_dtype),
                normal((n, w.H, inter), w.w_std, w.w_dtype))

    out = dict(x=[], router_w=[], router_b=[], w_gate=[], w_up=[], w_down=[],
               ws_gate=[], ws_up=[], ws_down=[])
    for _ in range(copies):
        out["x"].append(normal((w.T, w.H), 1.0, w.x_dtype))
        out["router_w"].append(normal((w.E, w.H), w.w_std, w.r_dtype))
        out["router_b"].append(
            torch.from_numpy(zipf_bias(w.E, w.zipf_s)).to(device) if w.zipf_s is not None else None)
        g, u, d = stack(w.E, w.I)
        out["w_gate"].append(g)
        out["w_up"].append(u)
        out["w_down"].append(d)
        if w.S > 0:
            sg, su, sd = stack(w.S, w.Is)
        else:
            sg = su = sd = None
        out["ws_gate"].append(sg)
        out["ws_up"].append(su)
        out["ws_down"].append(sd)
    if copies == 1:
        return {k: v[0] for k, v in out.items()}
    return out


def to_torch(inputs: dict, device="cuda") -> dict:
    """Move a ``make_inputs`` dict to torch tensors on ``device`` (bits preserved)."""
    import torch

    def conv(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {k: conv(v) for k, v in inputs.items()}


def from_torch(inputs: dict) -> dict:
    """Bring torch tensors back to numpy arrays of stored bits (for the oracle)."""
    import torch

    def conv(t):
        if t is None:
            return None
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    return {k: conv(v) for k, v in inputs.items()}
