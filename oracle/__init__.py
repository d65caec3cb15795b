"""CPU oracle for the quantized MoE FFN layer (ctypes wrapper around moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it to produce expected values. The product library never imports,
links or runs anything here, and nothing here touches the GPU library.

Functions take the canonical-layout arrays that ``quantized_moe_bit_amd.synth``
produces and return NumPy arrays. See moe_oracle.c for what each one computes
and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

STACK_EPS = 1e-6


def build() -> str:
    """Compile moe_oracle.c with gcc (fp32 router order needs no contraction and no fast-math)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _QMat(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p), ("q4_0", C.c_int)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int
        L.orc_set_threads.argtypes = [i32]
        L.orc_get_threads.restype = i32
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_gelu_tanh.argtypes = [C.c_double]
        L.orc_gelu_tanh.restype = C.c_double
        L.orc_dequant_row.argtypes = [i32, i32, vp, vp, vp, vp]
        L.orc_dequant_q4_0_row.argtypes = [i32, vp, vp]
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_router_logits.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.orc_topk.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.orc_router_prologue.argtypes = [i32, i32, vp, vp, C.c_double, vp]
        L.orc_bucket.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_ffn.argtypes = [i32, i32, vp, C.POINTER(_QMat), C.POINTER(_QMat), C.POINTER(_QMat), vp]
        L.orc_layer_tokens.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, vp] + \
            [C.POINTER(_QMat)] * 6 + [vp, vp, vp, vp, vp]
        L.orc_stack_glue.argtypes = [i32, i32, vp, vp, vp, C.c_double, C.c_double, vp, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def f64_to_bf16(v: float) -> int:
    return int(lib().orc_f64_to_bf16(float(v)))


def gelu_tanh(v: float) -> float:
    return float(lib().orc_gelu_tanh(float(v)))


def dequant_row(bits: int, codes, scales, biases, K: int) -> np.ndarray:
    out = np.empty(K, np.float64)
    codes, scales, biases = _c(codes, np.uint8), _c(scales, np.uint16), _c(biases, np.uint16)
    lib().orc_dequant_row(bits, K, _p(codes), _p(scales), _p(biases), _p(out))
    return out


def f16_to_f64(bits: int) -> float:
    return float(lib().orc_f16_to_f64(int(bits)))


def dequant_q4_0_row(blocks, K: int) -> np.ndarray:
    """One row of K elements from K/32 Q4_0 blocks (uint8, 18 bytes each)."""
    out = np.empty(K, np.float64)
    blocks = _c(blocks, np.uint8)
    lib().orc_dequant_q4_0_row(K, _p(blocks), _p(out))
    return out


def router_logits(x, rq, rs, rb, logit_bias=None) -> np.ndarray:
    """x: bf16 bits [T,d]; rq: uint8 [E,d]; rs, rb: bf16 bits [E,d/64] -> fp32 [T,E]."""
    x, rq, rs, rb = _c(x, np.uint16), _c(rq, np.uint8), _c(rs, np.uint16), _c(rb, np.uint16)
    T, d = x.shape
    E = rq.shape[0]
    lb = None if logit_bias is None else _c(logit_bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(T, d, E, _p(x), _p(rq), _p(rs), _p(rb), _p(lb), _p(out))
    return out


def topk(logits, k: int, per_expert_scale=None):
    """-> (idx int32 [T,k], w float64 [T,k]); per_expert_scale: optional bf16 bits [E]"""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    pes = None if per_expert_scale is None else _c(per_expert_scale, np.uint16)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_topk(T, E, k, _p(logits), _p(pes), _p(idx), _p(w))
    return idx, w


def router_prologue(x, router_scale, eps: float = STACK_EPS):
    """x: bf16 bits [T,d]; router_scale: bf16 bits [d] -> router input u, bf16 bits [T,d]"""
    x = _c(x, np.uint16)
    rs = _c(router_scale, np.uint16)
    T, d = x.shape
    u = np.empty_like(x)
    lib().orc_router_prologue(T, d, _p(x), _p(rs), float(eps), _p(u))
    return u


def bucket(idx, E: int):
    """-> (counts [E], offsets [E+1], perm [T*k], pos [T*k]) all int32"""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    lib().orc_bucket(T, E, k, _p(idx), _p(counts), _p(offsets), _p(perm), _p(pos))
    return counts, offsets, perm, pos


class _Keep:
    """Holds contiguous copies alive while a ctypes struct points into them."""

    def __init__(self):
        self.refs = []

    def qmat(self, m) -> _QMat:
        if getattr(m, "fmt", "affine") == "q4_0":
            c = _c(m.codes, np.uint8)
            self.refs.append(c)
            return _QMat(_p(c), None, None, 1)
        c, s, b = _c(m.codes, np.uint8), _c(m.scales, np.uint16), _c(m.biases, np.uint16)
        self.refs += [c, s, b]
        return _QMat(_p(c), _p(s), _p(b), 0)


def ffn(x_f64, gate, up, down) -> np.ndarray:
    """One expert (QMat views of a single expert) on one float64 token vector."""
    keep = _Keep()
    x = _c(x_f64, np.float64)
    d = x.shape[0]
    I = gate.out_dim
    r = np.empty(d, np.float64)
    lib().orc_ffn(d, I, _p(x), C.byref(keep.qmat(gate)), C.byref(keep.qmat(up)),
                  C.byref(keep.qmat(down)), _p(r))
    return r


def layer_tokens(layer, x, idx, w, tokens: Optional[Sequence[int]] = None, want_parts=False):
    """Layer output (float64) for the listed tokens of x (bf16 bits [T,d]) under routing idx/w.
    want_parts: also the ungated shared output, the per-slot outputs and the shared-expert
    gate values (1 without a gate)."""
    dims = layer.dims
    x = _c(x, np.uint16)
    T, d = x.shape
    toks = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    n = toks.shape[0]
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    keep = _Keep()
    y = np.empty((n, d), np.float64)
    sh = np.empty((n, d), np.float64) if want_parts else None
    r = np.empty((n, dims.top_k, d), np.float64) if want_parts else None
    a = np.empty(n, np.float64) if want_parts else None
    sg = getattr(layer, "shared_gate", None)
    sg = None if sg is None else _c(sg, np.uint16)
    qs = [keep.qmat(m) for m in (layer.gate, layer.up, layer.down, layer.sh_gate, layer.sh_up, layer.sh_down)]
    lib().orc_layer_tokens(d, dims.n_experts, dims.top_k, dims.d_expert, dims.d_shared, _p(x), n,
                           _p(toks), _p(idx), _p(w), *[C.byref(q) for q in qs], _p(sg), _p(y), _p(sh), _p(r),
                           _p(a))
    if want_parts:
        return y, sh, r, a
    return y


def route(layer, x):
    """Router logits, top-k and weights, and expert grouping for all tokens of x (with the
    router prologue and per-expert scale when the layer has them)."""
    u = x if layer.router_scale is None else router_prologue(x, layer.router_scale)
    logits = router_logits(u, layer.router.codes, layer.router.scales, layer.router.biases,
                           layer.logit_bias)
    idx, w = topk(logits, layer.dims.top_k, layer.per_expert_scale)
    counts, offsets, perm, pos = bucket(idx, layer.dims.n_experts)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, pos=pos)


def layer_forward(layer, x, tokens: Optional[Sequence[int]] = None):
    """Route every token, then the layer output for the listed tokens (all by default)."""
    r = route(layer, x)
    y = layer_tokens(layer, x, r["idx"], r["w"], tokens)
    return y, r


def stack_glue(h, y, eps: float = STACK_EPS, post=None, scalar: float = 1.0):
    """-> (h_next, x_next) bf16 bits [T,d]; y float64 [T,d] or None (first layer's norm only);
    post: optional bf16 bits [d] (post-FFN norm weight), scalar: layer scalar (with y)."""
    h = _c(h, np.uint16)
    T, d = h.shape
    yy = None if y is None else _c(y, np.float64)
    pp = None if post is None else _c(post, np.uint16)
    hn = np.empty_like(h)
    xn = np.empty_like(h)
    lib().orc_stack_glue(T, d, _p(h), _p(yy), _p(pp), float(scalar), float(eps), _p(hn), _p(xn))
    return hn, xn
