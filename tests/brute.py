"""Independent dense brute force of the quantized MoE layer, for tiny layers only.

Written separately from the oracle (no shared code) and structured differently:
it dequantizes whole weight tensors with NumPy, evaluates *every* expert on
*every* token, picks experts with a full sort, and masks. Its bf16 rounding
helper (exact rational round-to-nearest-even via ``fractions``) pins the
oracle's rounding. It is used to pin the oracle, never the GPU path directly.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16_exact(v: float) -> float:
    """Exact round-to-nearest-even of a finite double to 8 significant bits (normal range)."""
    if v == 0.0 or not math.isfinite(v):
        return v
    f = Fraction(v)
    a = abs(f)
    e = math.floor(math.log2(a))
    # fix possible off-by-one from log2 rounding
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # below the normal range the quantum stays 2^-133
    q = Fraction(2) ** (e - 7)            # spacing of 8-significant-bit values at this binade
    n = a / q
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = float(lo * q)
    return -r if f < 0 else r


def unpack_codes(codes: np.ndarray, bits: int, K: int) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    if bits == 8:
        return codes[..., :K].astype(np.int64)
    lo = codes & 0x0F
    hi = codes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    return q[..., :K].astype(np.int64)


def dense(m) -> np.ndarray:
    """Dequantize a QMat (possibly stacked) to float64 [..., out, in]."""
    if getattr(m, "fmt", "affine") == "q4_0":
        blk = np.asarray(m.codes, np.uint8).reshape(m.codes.shape[:-1] + (m.in_dim // 32, 18))
        d = np.ascontiguousarray(blk[..., :2]).view(np.float16)[..., 0].astype(np.float64)
        body = blk[..., 2:]
        q = np.concatenate([body & 0x0F, body >> 4], axis=-1).astype(np.int64)   # elements 0-15, 16-31
        return (d[..., None] * (q - 8)).reshape(m.codes.shape[:-1] + (m.in_dim,))
    q = unpack_codes(m.codes, m.bits, m.in_dim)
    s = np.repeat(bf16_value(m.scales), 64, axis=-1)
    b = np.repeat(bf16_value(m.biases), 64, axis=-1)
    return s * q + b


def rowdot(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Row-wise dot products with one summation routine for every row (np.sum)."""
    return np.sum(W * x[None, :], axis=-1)


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(v, np.float64)), approximate="tanh").numpy()


def ffn_dense(x: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    g = rowdot(Wg, x)
    u = rowdot(Wu, x)
    h = gelu_tanh(g) * u
    return rowdot(Wd, h)


def router_prologue(x: np.ndarray, rs: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Router input: x / rms(x) (no learned scale) * router_scale / sqrt(d), each value rounded
    exactly to bf16 (x, rs float64 [T, d] / [d] -> float64 values of the bf16 results)."""
    d = x.shape[-1]
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    v = x * inv * rs[None, :] / math.sqrt(d)
    return np.vectorize(rne_bf16_exact, otypes=[np.float64])(v)


def layer(lay, x_bits: np.ndarray):
    """-> dict(logits64, order, idx, w, y) computed densely for every token and expert."""
    dims = lay.dims
    x = bf16_value(x_bits)
    T = x.shape[0]
    E, k = dims.n_experts, dims.top_k
    Wr = dense(lay.router)
    Wg, Wu, Wd = dense(lay.gate), dense(lay.up), dense(lay.down)
    Sg, Su, Sd = dense(lay.sh_gate), dense(lay.sh_up), dense(lay.sh_down)
    xr = x if lay.router_scale is None else router_prologue(x, bf16_value(lay.router_scale))
    logits = np.stack([rowdot(Wr, xr[t]) for t in range(T)])
    if lay.logit_bias is not None:
        logits = logits + lay.logit_bias.astype(np.float64)[None, :]
    y = np.zeros((T, dims.d_model))
    idx = np.zeros((T, k), np.int64)
    wts = np.zeros((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))       # by value desc, then index asc
        sel = order[:k]
        z = np.exp(logits[t, sel] - logits[t, sel].max())
        wsel = z / z.sum()
        if lay.per_expert_scale is not None:
            wsel = wsel * bf16_value(lay.per_expert_scale)[sel]
        mask = np.zeros(E)
        mask[sel] = wsel
        outs = np.stack([ffn_dense(x[t], Wg[e], Wu[e], Wd[e]) for e in range(E)])  # every expert
        sh = ffn_dense(x[t], Sg, Su, Sd)
        if getattr(lay, "shared_gate", None) is not None:     # gated shared expert: sigmoid(g . x)
            z = float(np.dot(x[t], bf16_value(lay.shared_gate)))
            sh = sh / (1.0 + math.exp(-z))
        y[t] = sh + (mask[:, None] * outs).sum(axis=0)
        idx[t] = sel
        wts[t] = wsel
    return dict(logits64=logits, idx=idx, w=wts, y=y)
