"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins: the pages' codec definition and byte accounting,
exact integer arithmetic, a full sort, closed forms, a library GELU, and a dense
brute force (tests/brute.py) written independently of the oracle.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import synth
from tests import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 rounding
def test_bf16_rounding_matches_exact_rne():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)))
    # exact midpoints between adjacent bf16 values: ties must go to the even pattern
    for m in range(128, 256):
        vals.append((m + 0.5) * 2.0 ** -7)
        vals.append(-(m + 0.5) * 2.0 ** 3)
    vals += [1.0, -1.0, 255.5 * 2 ** -7, 2.0 ** -130, 3.5 * 2 ** -133, 1e-40, 0.0]
    for v in vals:
        got = oracle.f64_to_bf16(float(v))
        exp = brute.rne_bf16_exact(float(v))
        got_v = float(brute.bf16_value(np.array([got], np.uint16))[0])
        assert got_v == exp, (v, hex(got), got_v, exp)


# ----------------------------------------------------------------------------- codec
def _golden_groups():
    groups = {}
    for line in open(os.path.join(GOLD, "codec_groups.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, key, *vals = line.split()
        g = groups.setdefault(name, {})
        if key == "bits":
            g[key] = int(vals[0])
        elif key in ("scale", "bias"):
            g[key] = int(vals[0], 16)
        elif key == "bytes":
            g[key] = np.array([int(v, 16) for v in vals], np.uint8)
        elif key == "weights":
            g[key] = np.array([float(v) for v in vals])
    return groups


@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_codec_hand_built_groups(name):
    g = _golden_groups()[name]
    got = oracle.dequant_row(g["bits"], g["bytes"], np.array([g["scale"]], np.uint16),
                             np.array([g["bias"]], np.uint16), 64)
    np.testing.assert_array_equal(got, g["weights"])


def test_codec_group_boundaries():
    """Scales/biases switch exactly every 64 elements; 4-bit low nibble is the even element."""
    K = 256
    codes = np.zeros(K // 2, np.uint8)
    codes[0] = 0x21          # element 0 -> 1, element 1 -> 2
    codes[32] = 0x03         # element 64 -> 3 (first of group 1)
    codes[31] = 0x50         # element 63 -> 5 (last of group 0)
    scales = synth.f32_to_bf16_bits(np.array([1.0, 2.0, 4.0, 8.0], np.float32))
    biases = synth.f32_to_bf16_bits(np.array([0.0, 10.0, 100.0, 1000.0], np.float32))
    w = oracle.dequant_row(4, codes, scales, biases, K)
    assert w[0] == 1.0 and w[1] == 2.0 and w[63] == 5.0 and w[62] == 0.0
    assert w[64] == 2.0 * 3 + 10.0 and w[65] == 10.0
    assert w[128] == 100.0 and w[255] == 1000.0


def test_expert_blob_byte_accounting():
    """The canonical 4-bit g64 format reproduces the Mference expert blob size and totals."""
    kv = {}
    for line in open(os.path.join(GOLD, "expert_blob_bytes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        kv[k] = int(v)
    dims = synth.Dims(kv["d_model"], kv["n_experts"], 8, kv["d_expert"], 2112)
    rng = np.random.default_rng(0)
    per_expert = 0
    for out_dim, in_dim in ((dims.d_expert, dims.d_model),) * 2 + ((dims.d_model, dims.d_expert),):
        m = synth.uniform_qmat(rng, (), out_dim, in_dim, 4)
        per_expert += m.codes.nbytes + m.scales.nbytes + m.biases.nbytes
    page = kv["page"]
    blob = -(-per_expert // page) * page
    assert blob == kv["blob_bytes"]
    assert blob * kv["n_experts"] * kv["n_layers"] == kv["total_bytes"]


# ----------------------------------------------------------------------------- Q4_0 codec
def _golden_q4_0():
    def val(tok):
        if "*2^" in tok:
            a, e = tok.split("*2^")
            return float(a) * 2.0 ** int(e)
        return float(tok)
    blocks = {}
    for line in open(os.path.join(GOLD, "q4_0_blocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, key, *vals = line.split()
        b = blocks.setdefault(name, {})
        if key == "d":
            b[key] = int(vals[0], 16)
        elif key == "bytes":
            b[key] = [int(v, 16) for v in vals]
        else:
            b[key] = np.array([val(v) for v in vals])
    out = {}
    for name, b in blocks.items():
        raw = np.array([b["d"] & 0xFF, b["d"] >> 8] + b["bytes"], np.uint8)
        assert raw.shape == (18,) and b["weights"].shape == (32,)
        out[name] = (raw, b["weights"])
    return out


@pytest.mark.parametrize("name", ["P", "Q", "R", "S", "U"])
def test_q4_0_hand_built_blocks(name):
    raw, weights = _golden_q4_0()[name]
    np.testing.assert_array_equal(oracle.dequant_q4_0_row(raw, 32), weights)


def test_q4_0_blocks_follow_in_order():
    """A row of several blocks: block b covers elements 32 b .. 32 b + 31, each with its own d."""
    g = _golden_q4_0()
    names = ["Q", "P", "S", "R", "U", "P"]
    raw = np.concatenate([g[n][0] for n in names])
    np.testing.assert_array_equal(oracle.dequant_q4_0_row(raw, 32 * len(names)),
                                  np.concatenate([g[n][1] for n in names]))


def test_fp16_decoding_matches_library_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_q4_0_round_trip_of_a_block_quantizer():
    """Blocks made by the usual Q4_0 quantizer (d = the block's largest-magnitude value / -8,
    code = round(x / d) + 8 clamped to 0..15) dequantize to within |d| of every input."""
    rng = np.random.default_rng(5)
    K = 32 * 40
    x = rng.standard_normal(K) * np.exp(rng.uniform(-6, 3, K // 32)).repeat(32)
    raw = np.zeros((K // 32, 18), np.uint8)
    dd = np.zeros(K // 32)
    for b in range(K // 32):
        xb = x[32 * b: 32 * b + 32]
        amax = xb[np.argmax(np.abs(xb))]
        d16 = np.float16(amax / -8.0)
        dd[b] = float(d16)
        q = np.clip(np.rint(xb / dd[b]) + 8, 0, 15).astype(np.uint8)
        raw[b, :2] = np.array([d16]).view(np.uint8)
        raw[b, 2:] = q[:16] | (q[16:] << 4)
    w = oracle.dequant_q4_0_row(raw.reshape(-1), K)
    assert np.all(np.abs(w - x) <= np.abs(dd).repeat(32) * (1 + 2.0 ** -9))
    # the pin has teeth: the nibble halves swapped would miss by far more
    swapped = raw.copy()
    swapped[:, 2:] = (raw[:, 2:] >> 4) | (raw[:, 2:] << 4)
    w2 = oracle.dequant_q4_0_row(swapped.reshape(-1), K)
    assert np.max(np.abs(w2 - x) / np.abs(dd).repeat(32)) > 4


def test_q4_0_layer_matches_dense_brute_force():
    dims = synth.Dims(d_model=256, n_experts=8, top_k=3, d_expert=128, d_shared=192, expert_format="q4_0")
    lay = synth.gen_layer(dims, 31, router="normal", zipf_s=0.8)
    x, _, _ = synth.gen_tokens(dims, 4, 31)
    _cmp_layer(lay, x, 4)


def test_q4_0_layer_equals_affine_layer_with_the_same_weights():
    """Q4_0 blocks whose two halves of a 64-group share d are the affine format with scale d,
    bias -8 d (exact in bf16 when d has at most 8 significant bits): identical oracle outputs."""
    dims = synth.Dims(d_model=256, n_experts=6, top_k=2, d_expert=64, d_shared=128)
    lay = synth.gen_layer(dims, 33, router="normal")
    qdims = synth.Dims(d_model=256, n_experts=6, top_k=2, d_expert=64, d_shared=128, expert_format="q4_0")
    qlay = synth.gen_layer(qdims, 33, router="normal")
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        m = getattr(lay, name)
        sval = synth.bf16_bits_to_f32(m.scales)
        # biases -8 * scale exactly (bf16 keeps the scale's 8 significant bits)
        m.biases = synth.f32_to_bf16_bits(np.float32(-8.0) * sval)
        # the same weights as Q4_0: element 32 h + i of group g from the canonical nibbles
        q = np.stack([m.codes & 0x0F, m.codes >> 4], axis=-1).reshape(m.codes.shape[:-1] + (m.in_dim,))
        qb = q.reshape(q.shape[:-1] + (m.in_dim // 32, 32))
        d16 = sval.astype(np.float16).repeat(2, axis=-1)      # bf16 values are exact in fp16 here
        assert np.array_equal(d16.astype(np.float32), sval.repeat(2, axis=-1))
        blk = np.empty(qb.shape[:-1] + (18,), np.uint8)
        blk[..., :2] = d16[..., None].view(np.uint8)
        blk[..., 2:] = (qb[..., :16] | (qb[..., 16:] << 4)).astype(np.uint8)
        qm = getattr(qlay, name)
        qm.codes = blk.reshape(qm.codes.shape)
    x, _, _ = synth.gen_tokens(dims, 5, 33)
    ya, ra = oracle.layer_forward(lay, x)
    yq, rq = oracle.layer_forward(qlay, x)
    np.testing.assert_array_equal(ra["idx"], rq["idx"])
    np.testing.assert_array_equal(ya, yq)


# ----------------------------------------------------------------------------- router
def _dyadic_router_case(rng, T=3, E=5, d=128):
    """Inputs on which every fp32 operation of the router is exact."""
    x = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    q = rng.integers(0, 256, size=(E, d)).astype(np.uint8)
    s = np.float32(2.0) ** -rng.integers(3, 7, size=(E, d // 64)).astype(np.float32)
    b = -np.float32(2.0) ** -rng.integers(0, 3, size=(E, d // 64)).astype(np.float32)
    return x, q, s, b


def test_router_exact_integer_case():
    rng = np.random.default_rng(3)
    x, q, s, b = _dyadic_router_case(rng)
    xb = synth.f32_to_bf16_bits(x)
    sb, bb = synth.f32_to_bf16_bits(s), synth.f32_to_bf16_bits(b)
    bias = np.array([0.5, -0.25, 0.0, 1.0, -2.0], np.float32)
    got = oracle.router_logits(xb, q, sb, bb, bias)
    T, d = x.shape
    for t in range(T):
        for e in range(q.shape[0]):
            exact = Fraction(0)
            for i in range(d):
                w = Fraction(float(s[e, i // 64])) * int(q[e, i]) + Fraction(float(b[e, i // 64]))
                exact += Fraction(float(x[t, i])) * w
            exact += Fraction(float(bias[e]))
            assert Fraction(float(got[t, e])) == exact


def test_router_fp32_within_error_bound_of_fp64():
    w = synth.Workload("r", synth.Dims(512, 16, 4, 64, 64), tokens=8, seed=5)
    lay = synth.workload_layer(w)
    x, _, _ = synth.workload_tokens(w, lay)
    got = oracle.router_logits(x, lay.router.codes, lay.router.scales, lay.router.biases).astype(np.float64)
    Wr = brute.dense(lay.router)
    xv = brute.bf16_value(x)
    exact = xv @ Wr.T
    mag = np.abs(xv) @ np.abs(Wr).T + np.abs(xv) @ np.abs(brute.bf16_value(
        np.repeat(lay.router.biases, 64, axis=1))).T
    u = 2.0 ** -24
    bound = 2 * (64 + lay.dims.G + 4) * u * mag
    err = np.abs(got - exact)
    assert np.all(err <= bound), (err.max(), bound.min())
    # and the bound is tight enough to see a single dropped term
    assert np.median(np.abs(xv[:, :1] * Wr[:, 0][None, :]) / bound) > 10


def test_router_matches_brute_force_selection():
    w = synth.WORKLOADS["tiny"]
    lay = synth.workload_layer(w)
    x, _, _ = synth.workload_tokens(w, lay, T=32)
    r = oracle.route(lay, x)
    b = brute.layer(lay, x[:6])
    np.testing.assert_array_equal(r["idx"][:6], b["idx"])


# ----------------------------------------------------------------------------- router prologue / epilogue
def test_router_prologue_closed_form():
    # constant inputs: x / rms(x) = 1 up to eps, so u = bf16(router_scale / sqrt(d))
    d = 256
    one = synth.f32_to_bf16_bits(np.ones((2, d), np.float32))
    u = oracle.router_prologue(one, synth.f32_to_bf16_bits(np.ones(d, np.float32)))
    assert np.all(u == 0x3D80)                                   # 1/16 exactly
    three = synth.f32_to_bf16_bits(np.full((1, d), -3.0, np.float32))
    u = oracle.router_prologue(three, synth.f32_to_bf16_bits(np.full(d, 2.0, np.float32)))
    assert np.all(u == 0xBE00)                                   # -2/16 = -0.125
    # router_scale entering per channel
    rs = synth.f32_to_bf16_bits(np.where(np.arange(d) % 2 == 0, 1.0, 4.0).astype(np.float32))
    u = oracle.router_prologue(one, rs)
    assert np.all(u[:, 0::2] == 0x3D80) and np.all(u[:, 1::2] == 0x3E80)   # 1/16 and 4/16
    # inputs small enough that eps = 1e-6 matters: x = 2^-10, mean(x^2) = 2^-20
    tiny = synth.f32_to_bf16_bits(np.full((1, d), 2.0 ** -10, np.float32))
    u = oracle.router_prologue(tiny, synth.f32_to_bf16_bits(np.ones(d, np.float32)))
    want = brute.rne_bf16_exact(2.0 ** -10 / math.sqrt(2.0 ** -20 + 1e-6) / 16.0)
    assert np.all(brute.bf16_value(u) == want) and abs(want - 2.0 ** -10 * 1024 / 16) > 0.01


def test_router_prologue_matches_exact_rounding():
    rng = np.random.default_rng(12)
    T, d = 3, 192
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32) * 3)
    rs = synth.f32_to_bf16_bits(rng.uniform(0.25, 2.0, d).astype(np.float32))
    u = oracle.router_prologue(x, rs)
    ref = brute.router_prologue(brute.bf16_value(x), brute.bf16_value(rs))
    np.testing.assert_array_equal(brute.bf16_value(u), ref)


def test_per_expert_scale_multiplies_routing_weights():
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((40, 32)).astype(np.float32)
    idx0, w0 = oracle.topk(logits, 4)
    idx1, w1 = oracle.topk(logits, 4, np.full(32, 0x3F80, np.uint16))     # scale 1: unchanged
    np.testing.assert_array_equal(idx1, idx0)
    np.testing.assert_array_equal(w1, w0)
    idx2, w2 = oracle.topk(logits, 4, np.full(32, 0x4000, np.uint16))     # scale 2: doubled exactly
    np.testing.assert_array_equal(idx2, idx0)
    np.testing.assert_array_equal(w2, 2.0 * w0)
    pes = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, 32).astype(np.float32))
    idx3, w3 = oracle.topk(logits, 4, pes)
    np.testing.assert_array_equal(idx3, idx0)                           # selection is unaffected
    np.testing.assert_allclose(w3, w0 * brute.bf16_value(pes)[idx0], rtol=1e-15)


# ----------------------------------------------------------------------------- top-k
def test_topk_equals_full_sort_with_ties():
    rng = np.random.default_rng(7)
    T, E = 200, 128
    logits = rng.integers(-6, 6, size=(T, E)).astype(np.float32) * np.float32(0.5)   # many ties
    logits[:50] = rng.standard_normal((50, E)).astype(np.float32)
    for k in (1, 2, 8, 9, E):
        idx, w = oracle.topk(logits, k)
        for t in range(T):
            order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
            np.testing.assert_array_equal(idx[t], order[:k])


def test_softmax_weights_closed_forms():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((64, 16)).astype(np.float32) * 3
    idx, w = oracle.topk(logits, 2)
    l0 = logits[np.arange(64), idx[:, 0]].astype(np.float64)
    l1 = logits[np.arange(64), idx[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)
    idx, w = oracle.topk(logits, 8)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 1e-15)                     # listed largest first
    flat = np.zeros((1, 16), np.float32)
    idx, w = oracle.topk(flat, 8)
    np.testing.assert_array_equal(idx[0], np.arange(8))           # all tied: lowest indices
    np.testing.assert_allclose(w[0], 1.0 / 8, rtol=1e-15)


# ----------------------------------------------------------------------------- bucketing
def test_bucket_matches_lexsort_and_invariants():
    rng = np.random.default_rng(9)
    T, E, k = 300, 128, 8
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[:40] = np.arange(k)                   # a hot expert set
    counts, offsets, perm, pos = oracle.bucket(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    pairs = np.arange(T * k)
    ref = pairs[np.lexsort((pairs // k, idx.ravel()))]
    np.testing.assert_array_equal(perm, ref)
    np.testing.assert_array_equal(pos[perm], np.arange(T * k))
    np.testing.assert_array_equal(np.sort(perm), pairs)


# ----------------------------------------------------------------------------- GELU
def test_gelu_tanh_matches_library():
    xs = np.concatenate([np.linspace(-12, 12, 481), [0.0, 1.0, -1.0, 1e-8, 30.0, -30.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(v) for v in xs])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(30.0) == 30.0 and oracle.gelu_tanh(-30.0) == 0.0


# ----------------------------------------------------------------------------- layer
def _cmp_layer(lay, x, ntok):
    r = oracle.route(lay, x[:ntok])
    y = oracle.layer_tokens(lay, x[:ntok], r["idx"], r["w"])
    b = brute.layer(lay, x[:ntok])
    np.testing.assert_array_equal(r["idx"], b["idx"])
    # routing weights: softmax of fp32 logits vs fp64 logits. Each logit is within the router's
    # error bound B (the bound of test_router_fp32_within_error_bound_of_fp64), so each weight
    # is within a relative exp(2 max B) - 1 of the fp64 one.
    xv = brute.bf16_value(x[:ntok] if lay.router_scale is None else oracle.router_prologue(x[:ntok], lay.router_scale))
    mag = np.abs(xv) @ np.abs(brute.dense(lay.router)).T + np.abs(xv) @ np.abs(
        brute.bf16_value(np.repeat(lay.router.biases, 64, axis=1))).T
    bound = 2 * (64 + lay.dims.G + 4) * 2.0 ** -24 * mag
    bmax = np.take_along_axis(bound, r["idx"], axis=1).max(axis=1, keepdims=True)
    if lay.per_expert_scale is not None:   # the logit bound is relative to the softmax weights
        bmax = bmax * (1.0 + 2.0 ** -40)
    assert np.all(np.abs(r["w"] - b["w"]) <= b["w"] * np.expm1(2 * bmax) + 1e-15)
    assert np.max(bmax) < 1e-2   # under 2 % relative: a wrong weight or a dropped logit term shows
    scale = np.sqrt(np.mean(b["y"] ** 2))
    assert np.max(np.abs(y - b["y"])) <= 1e-5 * scale, np.max(np.abs(y - b["y"])) / scale
    return y, b


def test_layer_matches_dense_brute_force_tiny_workload():
    w = synth.WORKLOADS["tiny"]
    lay = synth.workload_layer(w)
    x, _, _ = synth.workload_tokens(w, lay)
    _cmp_layer(lay, x, w.tokens)


def test_layer_matches_dense_brute_force_odd_shapes():
    dims = synth.Dims(d_model=192, n_experts=5, top_k=3, d_expert=64, d_shared=128)
    lay = synth.gen_layer(dims, 21, router="normal", zipf_s=1.0)
    x, _, _ = synth.gen_tokens(dims, 3, 21)
    _cmp_layer(lay, x, 3)


def test_layer_matches_dense_brute_force_with_router_prologue_and_expert_scale():
    dims = synth.Dims(d_model=256, n_experts=8, top_k=3, d_expert=64, d_shared=128)
    lay = synth.gen_layer(dims, 23, router="normal")
    rng = np.random.default_rng(23)
    lay.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, dims.d_model).astype(np.float32))
    lay.per_expert_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, dims.n_experts).astype(np.float32))
    x, _, _ = synth.gen_tokens(dims, 4, 23)
    _cmp_layer(lay, x, 4)


def test_layer_matches_dense_brute_force_with_gated_shared_expert():
    """Gated shared expert (Mference system design, "Scope and limitations": the Qwen 3.6
    layers have one), read as the shared branch times sigmoid(g . x): against the brute force,
    which evaluates the gate with its own dot product and exp."""
    dims = synth.Dims(d_model=256, n_experts=16, top_k=4, d_expert=64, d_shared=64)
    lay = synth.gen_layer(dims, 25, router="normal")
    lay.shared_gate = synth.f32_to_bf16_bits(
        np.random.default_rng(25).normal(0, 1 / np.sqrt(dims.d_model), dims.d_model).astype(np.float32))
    x, _, _ = synth.gen_tokens(dims, 4, 25)
    _cmp_layer(lay, x, 4)


def test_shared_gate_closed_forms():
    """g = 0 gives a gate of exactly 1/2; g and -g give gates summing to 1 (so the two outputs
    sum to twice the g = 0 output); a gate driven to +-40 turns the shared branch fully on or
    off to float64 precision."""
    dims = synth.Dims(d_model=128, n_experts=8, top_k=2, d_expert=64, d_shared=128)
    lay = synth.gen_layer(dims, 61, router="normal")
    x, _, _ = synth.gen_tokens(dims, 4, 61)
    r = oracle.route(lay, x)
    y1, sh, _, a1 = oracle.layer_tokens(lay, x, r["idx"], r["w"], want_parts=True)
    routed = y1 - sh
    scale = np.abs(y1).max()

    def run(g):
        lay.shared_gate = g
        y, sh_g, _, a = oracle.layer_tokens(lay, x, r["idx"], r["w"], want_parts=True)
        np.testing.assert_array_equal(sh_g, sh)   # the ungated branch does not depend on g
        return y, a

    yz, az = run(np.zeros(dims.d_model, np.uint16))
    assert np.all(az == 0.5)
    np.testing.assert_allclose(yz, routed + 0.5 * sh, rtol=0, atol=1e-13 * scale)
    g = synth.f32_to_bf16_bits(np.random.default_rng(5).normal(0, 0.2, dims.d_model).astype(np.float32))
    yp, ap = run(g)
    yn, an = run(g ^ np.uint16(0x8000))
    assert np.all(np.abs(ap - 0.5) > 1e-3)
    np.testing.assert_allclose(ap + an, 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(yp + yn, 2 * yz, rtol=0, atol=1e-12 * scale)
    # against the library sigmoid of an independently formed dot product
    z = brute.bf16_value(x) @ brute.bf16_value(g)
    np.testing.assert_allclose(ap, torch.sigmoid(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=0)
    # saturation on token 0: z = +-40 (up to the bf16 rounding of g)
    x0 = brute.bf16_value(x[0])
    gs = synth.f32_to_bf16_bits((40.0 * x0 / np.dot(x0, x0)).astype(np.float32))
    yon, aon = run(gs)
    yoff, aoff = run(gs ^ np.uint16(0x8000))
    assert aon[0] > 1 - 1e-16 and aoff[0] < 1e-16
    np.testing.assert_allclose(yon[0], y1[0], rtol=0, atol=1e-14 * scale)
    np.testing.assert_allclose(yoff[0], routed[0], rtol=0, atol=1e-14 * scale)
    lay.shared_gate = None


def test_identical_experts_make_output_independent_of_routing():
    dims = synth.Dims(d_model=128, n_experts=6, top_k=2, d_expert=64, d_shared=64)
    lay = synth.gen_layer(dims, 31, router="uniform")
    for m in (lay.gate, lay.up, lay.down):
        m.codes[:] = m.codes[0]
        m.scales[:] = m.scales[0]
        m.biases[:] = m.biases[0]
    x, _, _ = synth.gen_tokens(dims, 5, 31)
    y1, r1 = oracle.layer_forward(lay, x)
    lay.router.codes[:] = np.random.default_rng(1).integers(0, 256, lay.router.codes.shape, dtype=np.uint8)
    y2, r2 = oracle.layer_forward(lay, x)
    assert not np.array_equal(r1["idx"], r2["idx"])
    scale = np.sqrt(np.mean(y1 ** 2))
    assert np.max(np.abs(y1 - y2)) <= 1e-13 * scale


def test_shared_branch_added_without_weight():
    dims = synth.Dims(d_model=128, n_experts=4, top_k=2, d_expert=64, d_shared=128)
    lay = synth.gen_layer(dims, 41, router="uniform")
    x, _, _ = synth.gen_tokens(dims, 3, 41)
    y_full, sh, r, a = oracle.layer_tokens(lay, x, *oracle.topk(oracle.route(lay, x)["logits"], 2),
                                           want_parts=True)
    assert np.all(a == 1.0)   # no shared-expert gate
    # shared part equals the dense brute force of the shared expert alone, unscaled
    for t in range(3):
        ref = brute.ffn_dense(brute.bf16_value(x[t]), brute.dense(lay.sh_gate), brute.dense(lay.sh_up),
                              brute.dense(lay.sh_down))
        np.testing.assert_allclose(sh[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # zero routed down projections: output is exactly the shared branch
    lay.down.scales[:] = 0
    lay.down.biases[:] = 0
    y0 = oracle.layer_forward(lay, x)[0]
    np.testing.assert_array_equal(y0, sh)


def test_constructed_ties_pick_lowest_indices():
    dims = synth.Dims(d_model=512, n_experts=40, top_k=8, d_expert=64, d_shared=64)
    lay = synth.gen_layer(dims, 51, router="normal", zipf_s=1.3, tie_groups=True)
    x, tied, grp = synth.gen_tokens(dims, 50, 51, layer=lay, tie_frac=0.1)
    r = oracle.route(lay, x)
    assert len(tied) == 5
    for t, g in zip(tied, grp):
        members = lay.tie_groups[g]
        lg = r["logits"][t]
        assert np.all(lg[members] == lg[members[0]])               # bit-equal logits
        order = np.sort(lg)[::-1]
        assert order[7] == order[8]                                  # ranks 8 and 9 tie
        full = np.lexsort((np.arange(dims.n_experts), -lg.astype(np.float64)))
        np.testing.assert_array_equal(r["idx"][t], full[:8])
        kept = np.intersect1d(r["idx"][t], members)
        np.testing.assert_array_equal(kept, members[:len(kept)])    # lowest indices kept
        assert len(kept) < 9
    # brute force (fp64, its own summation) agrees on the tied tokens' selection
    b = brute.layer(lay, x[tied[:2]])
    np.testing.assert_array_equal(b["idx"], r["idx"][tied[:2]])


def test_threads_do_not_change_results():
    w = synth.Workload("t", synth.Dims(256, 16, 4, 64, 128), tokens=24, seed=61)
    lay = synth.workload_layer(w)
    x, _, _ = synth.workload_tokens(w, lay)
    n0 = oracle.get_threads()
    try:
        oracle.set_threads(1)
        y1, r1 = oracle.layer_forward(lay, x)
        oracle.set_threads(max(2, n0))
        y2, r2 = oracle.layer_forward(lay, x)
    finally:
        oracle.set_threads(n0)
    np.testing.assert_array_equal(r1["logits"], r2["logits"])
    np.testing.assert_array_equal(y1, y2)


# ----------------------------------------------------------------------------- stack glue
def test_stack_glue_closed_forms():
    d = 256
    h = synth.f32_to_bf16_bits(np.full((1, d), 3.0, np.float32))
    y = np.full((1, d), 1.0)
    hn, xn = oracle.stack_glue(h, y, eps=0.0)
    assert np.all(brute.bf16_value(hn) == 4.0)
    assert np.all(brute.bf16_value(xn) == 1.0)                 # constant vector normalizes to 1
    rng = np.random.default_rng(71)
    h = synth.f32_to_bf16_bits(rng.standard_normal((4, d)).astype(np.float32) * 5)
    y = rng.standard_normal((4, d))
    hn, xn = oracle.stack_glue(h, y)
    ref_h = brute.bf16_value(h) + y
    for t in range(4):
        for i in range(0, d, 17):
            assert float(brute.bf16_value(hn[t, i])) == brute.rne_bf16_exact(float(ref_h[t, i]))
    xv = brute.bf16_value(xn)
    np.testing.assert_allclose(np.sqrt(np.mean(xv ** 2, axis=1)), 1.0, rtol=4e-3)


def test_stack_glue_layer_tail():
    # post-FFN norm, residual add and layer scalar (Mference "Decode", cb2)
    d = 128
    rng = np.random.default_rng(72)
    post = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, d).astype(np.float32))
    zero = np.zeros((1, d), np.uint16)
    # a constant layer output normalizes to 1: h_next = post (h = 0, scalar 1)
    hn, _ = oracle.stack_glue(zero, np.full((1, d), -7.0), post=post)
    np.testing.assert_array_equal(brute.bf16_value(hn)[0], -brute.bf16_value(post))
    # the scalar multiplies the whole stream after the add: 2 doubles it exactly
    h = synth.f32_to_bf16_bits(rng.standard_normal((3, d)).astype(np.float32) * 4)
    y = rng.standard_normal((3, d)) * 3
    h1, _ = oracle.stack_glue(h, y, post=post, scalar=1.0)
    h2, _ = oracle.stack_glue(h, y, post=post, scalar=2.0)
    np.testing.assert_array_equal(brute.bf16_value(h2), 2.0 * brute.bf16_value(h1))
    # against an independent float64 computation rounded exactly
    s = 0.75
    hn, xn = oracle.stack_glue(h, y, post=post, scalar=s)
    z = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + 1e-6) * brute.bf16_value(post)[None, :]
    ref = (brute.bf16_value(h) + z) * s
    for t in range(3):
        for i in range(0, d, 7):
            assert float(brute.bf16_value(hn[t, i])) == brute.rne_bf16_exact(float(ref[t, i]))
    # no post weight and scalar 1: the plain residual step
    hp, xp = oracle.stack_glue(h, y)
    hq, xq = oracle.stack_glue(h, y, post=None, scalar=1.0)
    np.testing.assert_array_equal(hp, hq)
    np.testing.assert_array_equal(xp, xq)
