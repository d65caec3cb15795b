"""Seeded synthetic inputs for the quantized MoE FFN layer.

This module only draws random numbers and lays them out in the canonical
byte layout. It holds none of the layer's arithmetic: no dequantization, no
matrix products, no routing. Both the CPU oracle and the GPU library consume
what it produces, so parity tests compare the two on identical bytes.

Canonical layout (the format every consumer reads):

* a weight matrix ``[out, in]`` is stored row-major;
* 4-bit codes are packed two per byte (so eight per little-endian u32), the
  lower-indexed element in the low nibble; 8-bit codes are one per byte;
* scales and biases are bf16 bit patterns ``uint16[out, in/64]``;
* routed experts are stacked along a leading ``[E, ...]`` axis.

The quantization scheme is the group-64 affine one the Mference system
design describes ("Why the runtime has this shape"): a weight is
``scale * code + bias`` with a BF16 scale and a BF16 bias per group of 64,
8-bit codes for the router and 4-bit codes for the shared and routed experts.

Expert matrices may instead be Q4_0 (Gem native architecture, "M4 Max operating
assumptions": 32 elements in an 18-byte block). A Q4_0 matrix ``[out, in]`` is
``uint8[..., out, in/32, 18]``: per block an fp16 scale d (little-endian), then 16
bytes whose byte j holds element j in its low nibble and element j + 16 in its
high nibble; the element's value is d * (code - 8). Its ``scales`` and
``biases`` arrays are empty.

Value distributions follow the five workloads the layer is measured on:
uniform codes, BF16 scale ~ U(0.002, 0.02), bias = -(code midpoint) * scale
+ N(0, 1e-3); router weights N(0, 0.02) quantized per group by min-max for the
2816-wide layer; activations bf16 N(0, 1); an optional Zipf(s) per-expert
logit bias; and optional groups of experts whose router rows agree on half of
the input width, used to give chosen tokens exactly tied top-8/top-9 logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

GROUP = 64


@dataclass(frozen=True)
class Dims:
    d_model: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    group: int = GROUP
    router_bits: int = 8
    expert_bits: int = 4
    expert_format: str = "affine"   # "affine" (group-64 scale/bias) or "q4_0" (32-element blocks)

    @property
    def G(self) -> int:
        return self.d_model // self.group


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    tokens: int
    seed: int
    router: str = "normal"          # "normal": N(0,0.02) min-max quantized; "uniform": uniform codes
    zipf_s: Optional[float] = None  # per-expert logit bias -s*ln(rank)
    tie_frac: float = 0.0           # fraction of tokens with exactly tied top-8/top-9 logits
    layers: int = 1
    shared_gate: bool = False       # gated shared expert (gate vector N(0, 1/d) in bf16)


TINY = Dims(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256)
GEMMA = Dims(d_model=2816, n_experts=128, top_k=8, d_expert=704, d_shared=2112)
GEMMA_Q4_0 = Dims(d_model=2816, n_experts=128, top_k=8, d_expert=704, d_shared=2112, expert_format="q4_0")
# Qwen 3.6 style layer: 256 routed experts, top-8, a gated shared expert, experts about half
# the size of the 2816-wide layer's (3 x 512 x 2048 against 3 x 704 x 2816 weights)
QWEN = Dims(d_model=2048, n_experts=256, top_k=8, d_expert=512, d_shared=512)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, tokens=4, seed=0, router="uniform"),
    # the same layer with the stated bias recipe (-8 * scale) applied to the 8-bit router as written
    "tiny_literal": Workload("tiny_literal", TINY, tokens=4, seed=0, router="uniform_mid8"),
    "decode": Workload("decode", GEMMA, tokens=1, seed=1),
    "stack": Workload("stack", GEMMA, tokens=256, seed=2, layers=30),
    "prefill512": Workload("prefill512", GEMMA, tokens=512, seed=3, zipf_s=1.1),
    "prefill4096": Workload("prefill4096", GEMMA, tokens=4096, seed=4, zipf_s=1.3, tie_frac=0.02),
    # the 2816-wide layer with Q4_0 experts
    "q4_0_decode": Workload("q4_0_decode", GEMMA_Q4_0, tokens=1, seed=7),
    "q4_0_prefill512": Workload("q4_0_prefill512", GEMMA_Q4_0, tokens=512, seed=8, zipf_s=1.1),
    "q4_0_prefill4096": Workload("q4_0_prefill4096", GEMMA_Q4_0, tokens=4096, seed=9, zipf_s=1.3, tie_frac=0.02),
    "qwen_decode": Workload("qwen_decode", QWEN, tokens=1, seed=5, shared_gate=True),
    "qwen_prefill4096": Workload("qwen_prefill4096", QWEN, tokens=4096, seed=6, zipf_s=1.3, tie_frac=0.02,
                                 shared_gate=True),
}

TIE_GROUP_SIZE = 9      # experts whose logits are made equal: ranks 8 and 9 tie
N_TIE_GROUPS = 4


# ----------------------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    # finite inputs: u + 0x8000 stays below 2^32, so 32-bit arithmetic cannot wrap
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- quantized matrices
@dataclass
class QMat:
    """One (or a stack of) quantized matrices in the canonical layout."""
    codes: np.ndarray   # uint8 [..., out, in*bits/8]; Q4_0: [..., out, in/32 * 18] blocks
    scales: np.ndarray  # uint16 [..., out, in/64]; Q4_0: [..., out, 0]
    biases: np.ndarray  # uint16 [..., out, in/64]; Q4_0: [..., out, 0]
    bits: int
    out_dim: int
    in_dim: int
    fmt: str = "affine"


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *key]))


def uniform_qmat(rng: np.random.Generator, lead: tuple, out_dim: int, in_dim: int, bits: int,
                 mid: Optional[int] = None, scale_range=(0.002, 0.02)) -> QMat:
    """Uniform codes, scale ~ U(scale_range), bias = -mid*scale + N(0, 1e-3) (noise scaled with the
    scale range), mid = 2^(bits-1) unless given."""
    G = in_dim // GROUP
    nbytes = in_dim * bits // 8
    shape = lead + (out_dim, nbytes)
    n = int(np.prod(shape))
    # uniform bytes drawn as 64-bit words (an order of magnitude faster than per-byte draws)
    codes = rng.integers(0, 1 << 64, size=(n + 7) // 8, dtype=np.uint64).view(np.uint8)[:n].reshape(shape)
    lo, hi = scale_range
    s = rng.random(size=lead + (out_dim, G), dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    s_bits = f32_to_bf16_bits(s)
    mid = np.float32(1 << (bits - 1) if mid is None else mid)
    noise = rng.standard_normal(size=lead + (out_dim, G), dtype=np.float32) * np.float32(1e-3 * hi / 0.02)
    b = -mid * bf16_bits_to_f32(s_bits) + noise
    return QMat(codes, s_bits, f32_to_bf16_bits(b), bits, out_dim, in_dim)


def q4_0_qmat(rng: np.random.Generator, lead: tuple, out_dim: int, in_dim: int,
              scale_range=(0.002, 0.02)) -> QMat:
    """Q4_0 blocks: uniform 4-bit codes, d = +-U(scale_range) (random sign) rounded to fp16."""
    nb = in_dim // 32
    shape = lead + (out_dim, nb)
    n = int(np.prod(shape)) * 16
    packed = rng.integers(0, 1 << 64, size=(n + 7) // 8, dtype=np.uint64).view(np.uint8)[:n]
    lo, hi = scale_range
    d = rng.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    d = np.where(rng.random(size=shape) < 0.5, -d, d).astype(np.float16)
    blocks = np.empty(shape + (18,), np.uint8)
    blocks[..., :2] = d.reshape(shape + (1,)).view(np.uint8)   # little-endian fp16
    blocks[..., 2:] = packed.reshape(shape + (16,))
    empty = np.zeros(lead + (out_dim, 0), np.uint16)
    return QMat(blocks.reshape(lead + (out_dim, nb * 18)), empty, empty.copy(), 4, out_dim, in_dim, "q4_0")


def expert_qmat(dims: Dims, rng: np.random.Generator, lead: tuple, out_dim: int, in_dim: int) -> QMat:
    if dims.expert_format == "q4_0":
        return q4_0_qmat(rng, lead, out_dim, in_dim)
    if dims.expert_format != "affine":
        raise ValueError(dims.expert_format)
    return uniform_qmat(rng, lead, out_dim, in_dim, dims.expert_bits)


def normal_router_qmat(rng: np.random.Generator, E: int, d: int, std: float = 0.02) -> QMat:
    """Router weights drawn N(0, std) and quantized to 8 bits per group of 64 by min-max."""
    G = d // GROUP
    w = rng.standard_normal(size=(E, G, GROUP), dtype=np.float32) * np.float32(std)
    mn = w.min(axis=-1)
    mx = w.max(axis=-1)
    s_bits = f32_to_bf16_bits((mx - mn) / np.float32(255.0))
    b_bits = f32_to_bf16_bits(mn)
    sf = bf16_bits_to_f32(s_bits)[..., None]
    bf = bf16_bits_to_f32(b_bits)[..., None]
    q = np.clip(np.rint((w - bf) / sf), 0, 255).astype(np.uint8)
    return QMat(q.reshape(E, d), s_bits, b_bits, 8, E, d)


@dataclass
class Layer:
    dims: Dims
    router: QMat
    gate: QMat
    up: QMat
    down: QMat
    sh_gate: QMat
    sh_up: QMat
    sh_down: QMat
    logit_bias: Optional[np.ndarray] = None       # float32 [E]
    tie_groups: Optional[np.ndarray] = None       # int32 [n_groups, 9], ascending within a group
    meta: dict = field(default_factory=dict)
    router_scale: Optional[np.ndarray] = None     # bf16 bits [d]: router prologue scale
    per_expert_scale: Optional[np.ndarray] = None  # bf16 bits [E]: routing-weight scale
    post_ffn_norm: Optional[np.ndarray] = None    # bf16 bits [d]: post-FFN norm weight (stack layer tail)
    layer_scalar: Optional[int] = None            # bf16 bits: layer scalar (stack layer tail)
    shared_gate: Optional[np.ndarray] = None      # bf16 bits [d]: shared-expert gate vector

    def nbytes(self) -> int:
        tot = 0
        for m in (self.router, self.gate, self.up, self.down, self.sh_gate, self.sh_up, self.sh_down):
            tot += m.codes.nbytes + m.scales.nbytes + m.biases.nbytes
        return tot


def gen_layer(dims: Dims, seed: int, *, router: str = "normal", zipf_s: Optional[float] = None,
              tie_groups: bool = False, layer_index: int = 0, shared_gate: bool = False) -> Layer:
    d, E, I, Is = dims.d_model, dims.n_experts, dims.d_expert, dims.d_shared
    key = (layer_index,)
    if router == "normal":
        rq = normal_router_qmat(_rng(seed, *key, 1), E, d)
    elif router == "uniform":
        rq = uniform_qmat(_rng(seed, *key, 1), (), E, d, dims.router_bits)
    elif router == "uniform_mid8":
        rq = uniform_qmat(_rng(seed, *key, 1), (), E, d, dims.router_bits, mid=8)
    else:
        raise ValueError(router)
    gate = expert_qmat(dims, _rng(seed, *key, 2), (E,), I, d)
    up = expert_qmat(dims, _rng(seed, *key, 3), (E,), I, d)
    down = expert_qmat(dims, _rng(seed, *key, 4), (E,), d, I)
    sh_gate = expert_qmat(dims, _rng(seed, *key, 5), (), Is, d)
    sh_up = expert_qmat(dims, _rng(seed, *key, 6), (), Is, d)
    sh_down = expert_qmat(dims, _rng(seed, *key, 7), (), d, Is)
    bias = None
    if zipf_s is not None:
        ranks = _rng(seed, *key, 8).permutation(E) + 1
        bias = (-np.float64(zipf_s) * np.log(ranks.astype(np.float64))).astype(np.float32)
    groups = None
    if tie_groups:
        if E < TIE_GROUP_SIZE * N_TIE_GROUPS or dims.top_k != TIE_GROUP_SIZE - 1:
            raise ValueError("tie groups need top_k = 8 and at least 36 experts")
        pick = _rng(seed, *key, 9).permutation(E)[: TIE_GROUP_SIZE * N_TIE_GROUPS]
        groups = np.sort(pick.reshape(N_TIE_GROUPS, TIE_GROUP_SIZE), axis=1).astype(np.int32)
        half_codes = d * dims.router_bits // 8 // 2
        half_groups = dims.G // 2
        for grp in groups:
            lead = grp[0]
            for e in grp[1:]:
                rq.codes[e, :half_codes] = rq.codes[lead, :half_codes]
                rq.scales[e, :half_groups] = rq.scales[lead, :half_groups]
                rq.biases[e, :half_groups] = rq.biases[lead, :half_groups]
                if bias is not None:
                    bias[e] = bias[lead]
    lay = Layer(dims, rq, gate, up, down, sh_gate, sh_up, sh_down, bias, groups,
                meta=dict(seed=seed, router=router, zipf_s=zipf_s, layer_index=layer_index))
    if shared_gate:   # g . x ~ N(0, 1) for unit-rms x
        g = _rng(seed, *key, 10).normal(0.0, 1.0 / np.sqrt(d), d).astype(np.float32)
        lay.shared_gate = f32_to_bf16_bits(g)
    return lay


def gen_tokens(dims: Dims, T: int, seed: int, *, layer: Optional[Layer] = None,
               tie_frac: float = 0.0, stream: int = 100) -> tuple:
    """Activations bf16 N(0,1) as uint16 bits [T, d]; returns (x, tied_token_ids, tied_group_ids).

    A tied token is zero on the upper half of the input width and, on the lower half, carries
    |N(0,1)| with the sign of (router code - code midpoint) of its tie group's shared row. The
    nine experts of the group then produce bit-identical logits for it (same codes, scales,
    biases and logit bias on the half where the token is non-zero), far above every other
    expert, so ranks 8 and 9 are tied by construction.
    """
    d = dims.d_model
    rng = _rng(seed, stream)
    x = f32_to_bf16_bits(rng.standard_normal(size=(T, d), dtype=np.float32))
    n_tie = int(round(tie_frac * T))
    tied = np.zeros(0, np.int32)
    tied_grp = np.zeros(0, np.int32)
    if n_tie:
        if layer is None or layer.tie_groups is None:
            raise ValueError("tied tokens need a layer built with tie groups")
        trng = _rng(seed, stream + 1)
        tied = np.sort(trng.permutation(T)[:n_tie]).astype(np.int32)
        tied_grp = (np.arange(n_tie) % layer.tie_groups.shape[0]).astype(np.int32)
        half = d // 2
        mid = 1 << (dims.router_bits - 1)
        for t, g in zip(tied, tied_grp):
            lead = layer.tie_groups[g][0]
            codes = layer.router.codes[lead, :half].astype(np.int32)   # 8-bit router: one code per byte
            sign = np.where(codes >= mid, 1.0, -1.0).astype(np.float32)
            mag = np.abs(trng.standard_normal(size=half, dtype=np.float32))
            row = np.zeros(d, np.float32)
            row[:half] = sign * mag
            x[t] = f32_to_bf16_bits(row)
    return x, tied, tied_grp


def gen_stack_tokens(dims: Dims, T: int, seed: int) -> np.ndarray:
    """Initial residual stream h_0, bf16 N(0,1) bits [T, d]."""
    rng = _rng(seed, 200)
    return f32_to_bf16_bits(rng.standard_normal(size=(T, dims.d_model), dtype=np.float32))


def workload_layer(w: Workload, layer_index: int = 0) -> Layer:
    return gen_layer(w.dims, w.seed, router=w.router, zipf_s=w.zipf_s,
                     tie_groups=w.tie_frac > 0, layer_index=layer_index, shared_gate=w.shared_gate)


def workload_tokens(w: Workload, layer: Optional[Layer] = None, T: Optional[int] = None):
    return gen_tokens(w.dims, w.tokens if T is None else T, w.seed, layer=layer, tie_frac=w.tie_frac)
