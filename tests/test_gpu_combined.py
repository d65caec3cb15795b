"""GPU parity with every optional layer feature at once, through the C ABI: a decode stack of
2048-wide layers with 256 experts (the gated-shared-expert workload's shape) whose layers carry
the router prologue and per-expert scale (Mference system design, "Decode", router listing),
the gated shared expert ("Scope and limitations") and the layer tail ("Decode", cb2), with
affine group-64 experts and with Q4_0 experts (Gem native architecture, "M4 Max operating
assumptions").

Layer by layer on the GPU's own stream (teacher forcing): logits bit-identical, top-k exact,
layer output within max |err| <= 2e-3 * rms of the oracle, residual step with the tail
bit-exact; then the stack entry point reproduces the layer-by-layer stream bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import binding as B
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

TOL = 2e-3


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def full_layer(dims, seed):
    lay = synth.gen_layer(dims, seed, router="normal", shared_gate=True)
    rng = np.random.default_rng(seed + 500)
    lay.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, dims.d_model).astype(np.float32))
    lay.per_expert_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, dims.n_experts).astype(np.float32))
    lay.post_ffn_norm = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, dims.d_model).astype(np.float32))
    lay.layer_scalar = int(synth.f32_to_bf16_bits(np.array([rng.uniform(0.6, 1.3)], np.float32))[0])
    return lay


@pytest.mark.parametrize("fmt", ["affine", "q4_0"])
def test_stack_with_every_layer_feature(fmt):
    dims = dataclasses.replace(synth.WORKLOADS["qwen_decode"].dims, expert_format=fmt)
    NL, T = 3, 4
    layers = [full_layer(dims, 120 + l) for l in range(NL)]
    dls = [DeviceLayer(l, max_tokens=16) for l in layers]
    h0 = synth.gen_stack_tokens(dims, T, 121)
    dev = torch.device("cuda:0")
    hs = tokens_to_device(h0, dev)
    xs = torch.empty_like(hs)
    ys = torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    B.moe_stack_glue(hs, None, hs, xs, T, dims.d_model)
    for l, (lay, dl) in enumerate(zip(layers, dls)):
        torch.cuda.synchronize()
        x_l = bits(xs)
        ref = oracle.route(lay, x_l)
        r = dl.route(xs)
        dl.decode(xs, ys)
        h_prev = bits(hs)
        post, scalar = dl.tail()
        B.moe_stack_glue(hs, ys, hs, xs, T, dims.d_model, post=post, scalar=scalar)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32),
                                      err_msg=f"layer {l} logits")
        np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"], err_msg=f"layer {l} top-k")
        y_ref = oracle.layer_tokens(lay, x_l, ref["idx"], ref["w"])
        y_gpu = ys.cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(y_ref ** 2))
        err = np.max(np.abs(y_gpu - y_ref)) / rms
        assert err <= TOL, f"layer {l}: max|err| {err:.2e} rms"
        scal = float(synth.bf16_bits_to_f32(np.array([lay.layer_scalar], np.uint16))[0])
        hn_ref, xn_ref = oracle.stack_glue(h_prev, y_gpu, post=lay.post_ffn_norm, scalar=scal)
        np.testing.assert_array_equal(bits(hs), hn_ref, err_msg=f"layer {l} residual")
        np.testing.assert_array_equal(bits(xs), xn_ref, err_msg=f"layer {l} norm")
        print(f"[combined] {fmt} layer {l}: logits and top-k exact, max|err| {err:.2e} rms, residual bit-exact",
              flush=True)
    h = tokens_to_device(h0, dev)
    xb = torch.empty((1, dims.d_model), dtype=torch.int16, device=dev)
    yb = torch.empty((1, dims.d_model), dtype=torch.float32, device=dev)
    hb = torch.empty_like(xb)
    for t in range(T):
        B.moe_stack_forward_decode([d.handle for d in dls], h[t:t + 1], 1, xb, yb, hb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(h), bits(hs))
    print(f"[combined] {fmt} stack entry point: {T} tokens x {NL} layers identical", flush=True)
    for d in dls:
        d.close()
