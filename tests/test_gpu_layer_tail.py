"""GPU parity of the layer tail in the decode stack (Mference system design, "Decode", cb2:
post-FFN norm, residual add, layer scalar), through the C ABI.

Layers carry an optional post-FFN norm weight and layer scalar (both, either one, or both
again on the last layer, whose tail the stack's final residual step applies). Layer by
layer, on the GPU's own stream (teacher forcing): top-k sets bit-exact, layer outputs within
max |err| <= 2e-3 * rms, and the residual step with the tail,
  h' = bf16((h + (y / rms(y)) * post) * scalar),  x = bf16(h' / rms(h')),
bit-exact against the oracle on the GPU's y (both sides round the fp64 value once). The
stack entry point then gives the same bits one token per call (residual step inside the
router launch) and with all tokens in one call (residual step in its own launch).
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import binding as B
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

TOL = 2e-3
DIMS = synth.Dims(d_model=2048, n_experts=16, top_k=4, d_expert=128, d_shared=256)
# (post-FFN norm, layer scalar) per layer
TAILS = [(True, True), (True, False), (False, True), (True, True)]


def say(msg):
    print(f"[tail] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def with_tail(seed, post, scalar):
    lay = synth.gen_layer(DIMS, seed, router="normal")
    rng = np.random.default_rng(seed + 2000)
    if post:
        lay.post_ffn_norm = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, DIMS.d_model).astype(np.float32))
    if scalar:
        lay.layer_scalar = int(synth.f32_to_bf16_bits(np.array([rng.uniform(0.6, 1.3)], np.float32))[0])
    return lay


def scalar_of(lay) -> float:
    if lay.layer_scalar is None:
        return 1.0
    return float(synth.bf16_bits_to_f32(np.array([lay.layer_scalar], np.uint16))[0])


def test_stack_with_layer_tail():
    T = 12   # T * d above the router launch's LDS budget: the all-tokens call takes the separate step
    layers = [with_tail(80 + l, *TAILS[l]) for l in range(len(TAILS))]
    dls = [DeviceLayer(l, max_tokens=16) for l in layers]
    h0 = synth.gen_stack_tokens(DIMS, T, 81)
    dev = torch.device("cuda:0")
    hs = tokens_to_device(h0, dev)
    xs = torch.empty_like(hs)
    ys = torch.empty((T, DIMS.d_model), dtype=torch.float32, device=dev)
    B.moe_stack_glue(hs, None, hs, xs, T, DIMS.d_model)
    for l, (lay, dl) in enumerate(zip(layers, dls)):
        torch.cuda.synchronize()
        x_l = bits(xs)
        ref = oracle.route(lay, x_l)
        r = dl.route(xs)
        dl.decode(xs, ys)
        h_prev = bits(hs)
        post, scalar = dl.tail()
        B.moe_stack_glue(hs, ys, hs, xs, T, DIMS.d_model, post=post, scalar=scalar)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"], err_msg=f"layer {l} top-k")
        y_ref = oracle.layer_tokens(lay, x_l, ref["idx"], ref["w"])
        y_gpu = ys.cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(y_ref ** 2))
        err = np.max(np.abs(y_gpu - y_ref)) / rms
        assert err <= TOL, f"layer {l}: max|err| {err:.2e} rms"
        hn_ref, xn_ref = oracle.stack_glue(h_prev, y_gpu, post=lay.post_ffn_norm, scalar=scalar_of(lay))
        np.testing.assert_array_equal(bits(hs), hn_ref, err_msg=f"layer {l} residual with tail")
        np.testing.assert_array_equal(bits(xs), xn_ref, err_msg=f"layer {l} norm")
        plain, _ = oracle.stack_glue(h_prev, y_gpu)
        assert not np.array_equal(plain, hn_ref)   # the tail changes the stream
        say(f"layer {l} tail {TAILS[l]}: top-k exact, max|err| {err:.2e} rms, residual and norm bit-exact")
    handles = [d.handle for d in dls]
    # one token per call: the residual step with the previous layer's tail runs in the router launch
    h = tokens_to_device(h0, dev)
    xb = torch.empty((1, DIMS.d_model), dtype=torch.int16, device=dev)
    yb = torch.empty((1, DIMS.d_model), dtype=torch.float32, device=dev)
    hb = torch.empty_like(xb)
    for t in range(T):
        B.moe_stack_forward_decode(handles, h[t:t + 1], 1, xb, yb, hb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(h), bits(hs))
    say(f"stack entry point, 1 token per call: {T} tokens x {len(TAILS)} layers identical")
    # all tokens in one call: separate residual launches
    hA = tokens_to_device(h0, dev)
    xA, hbA = torch.empty_like(hA), torch.empty_like(hA)
    yA = torch.empty((T, DIMS.d_model), dtype=torch.float32, device=dev)
    B.moe_stack_forward_decode(handles, hA, T, xA, yA, hbA)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(hA), bits(hs))
    np.testing.assert_array_equal(bits(xA), bits(xs))
    say(f"stack entry point, {T} tokens per call: identical")
    for d in dls:
        d.close()
