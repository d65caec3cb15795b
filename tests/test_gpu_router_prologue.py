"""GPU parity of the router prologue and per-expert scale (Mference system design, "Decode",
router listing), through the C ABI: layers created with router_scale and per_expert_scale.

The router reads u = bf16(((x / rms(x)) * router_scale) / sqrt(d)) instead of x, and every
routing weight is multiplied by its expert's scale. Same bar as the other parity tests:
logits bit-identical to the oracle's, top-k sets and grouping bit-exact, weights within 2e-6
relative, outputs within max |err| <= 2e-3 * rms; the decode stack entry point gives the same
bits as the layer-by-layer run.
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

SHAPES = {
    "w2816": (synth.WORKLOADS["decode"].dims, 300),
    "small": (synth.Dims(d_model=512, n_experts=16, top_k=4, d_expert=128, d_shared=256), 70),
    # 72 input groups, more than the group-split prefill router takes: the matrix-core router
    # reads the prologue's output, with its last 64-token block and 16-expert block part-filled
    "wide_matrix_router": (synth.Dims(d_model=4608, n_experts=24, top_k=4, d_expert=128, d_shared=128), 100),
}


def say(msg):
    print(f"[prologue] {msg}", flush=True)


def with_prologue(dims, seed):
    lay = synth.gen_layer(dims, seed, router="normal")
    rng = np.random.default_rng(seed + 1000)
    lay.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, dims.d_model).astype(np.float32))
    lay.per_expert_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, dims.n_experts).astype(np.float32))
    return lay


def check_route(dl, lay, x, what):
    r = dl.route(tokens_to_device(x))
    torch.cuda.synchronize()
    ref = oracle.route(lay, x)
    np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32),
                                  err_msg=f"{what} logits")
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"], err_msg=f"{what} top-k")
    np.testing.assert_allclose(r["w"].cpu().numpy(), ref["w"], rtol=2e-6, atol=1e-7, err_msg=f"{what} weights")
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(r["perm"].cpu().numpy(), ref["perm"])
    assert not np.allclose(ref["w"].sum(axis=1), 1.0)   # the per-expert scale is in effect
    return ref


def check_close(y, y_ref, what):
    y = np.asarray(y, np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y - y_ref))
    assert np.all(np.isfinite(y)) and err <= TOL * rms, f"{what}: max|err| {err / rms:.2e} rms"
    say(f"{what}: max|err| {err / rms:.2e} rms")


@pytest.mark.parametrize("name", list(SHAPES))
def test_layer_with_router_prologue(name):
    dims, T = SHAPES[name]
    lay = with_prologue(dims, 61)
    x, _, _ = synth.gen_tokens(dims, T, 62)
    dl = DeviceLayer(lay, max_tokens=T)
    ref = check_route(dl, lay, x, f"{name} route T={T}")          # prefill router
    check_route(dl, lay, x[:5], f"{name} route T=5")              # decode router
    say(f"{name}: logits bit-exact, top-k and grouping exact (T={T} and T=5)")
    y_ref = oracle.layer_tokens(lay, x, ref["idx"], ref["w"])
    xd = tokens_to_device(x)
    y = dl.prefill(xd)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref, f"{name} prefill T={T}")
    y = dl.decode(xd[:3])
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref[:3], f"{name} decode T=3")
    # 16 tokens: the decode router input no longer fits the router launch's LDS, so the
    # prologue runs as a launch of its own
    check_route(dl, lay, x[:16], f"{name} route T=16")
    y = dl.decode(xd[:16])
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref[:16], f"{name} decode T=16")
    dl.close()


def test_stack_with_router_prologue():
    dims = SHAPES["small"][0]
    NL, T = 3, 4
    layers = [with_prologue(dims, 70 + l) for l in range(NL)]
    dls = [DeviceLayer(l, max_tokens=16) for l in layers]
    h0 = synth.gen_stack_tokens(dims, T, 71)
    dev = torch.device("cuda:0")
    # layer by layer: glue, route + decode, per token
    hs = tokens_to_device(h0, dev)
    xs = torch.empty_like(hs)
    ys = torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    B.moe_stack_glue(hs, None, hs, xs, T, dims.d_model)
    for l in range(NL):
        torch.cuda.synchronize()
        x_l = xs.cpu().numpy().view(np.uint16)
        ref = oracle.route(layers[l], x_l)
        r = dls[l].route(xs)
        dls[l].decode(xs, ys)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"], err_msg=f"layer {l} top-k")
        y_ref = oracle.layer_tokens(layers[l], x_l, ref["idx"], ref["w"])
        check_close(ys.cpu().numpy(), y_ref, f"stack layer {l}")
        B.moe_stack_glue(hs, ys, hs, xs, T, dims.d_model)
    torch.cuda.synchronize()
    # the stack entry point, one token per call
    h = tokens_to_device(h0, dev)
    xb = torch.empty((1, dims.d_model), dtype=torch.int16, device=dev)
    yb = torch.empty((1, dims.d_model), dtype=torch.float32, device=dev)
    hb = torch.empty_like(xb)
    for t in range(T):
        B.moe_stack_forward_decode([d.handle for d in dls], h[t:t + 1], 1, xb, yb, hb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h.cpu().numpy().view(np.uint16), hs.cpu().numpy().view(np.uint16))
    say(f"stack entry point with the prologue: {T} tokens x {NL} layers identical to the layer-by-layer run")
    for d in dls:
        d.close()
