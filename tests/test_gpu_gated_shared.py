"""GPU parity of the gated shared expert on a Qwen 3.6 style layer (Mference system design,
"Scope and limitations": Qwen 3.6 layers have 256 experts and a shared branch behind a
gate), through the C ABI.

Layer: d_model 2048, 256 experts, top-8, expert width 512, shared width 512, 8-bit g64
router, 4-bit g64 experts, and a bf16 gate vector g: the shared branch is multiplied by
sigmoid(g . x) per token. Same bar as the other parity tests: logits bit-identical, top-k
and grouping bit-exact, outputs within max |err| <= 2e-3 * rms of the oracle, on every
token, including the 4096-token prefill chunk.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

TOL = 2e-3


def say(msg):
    print(f"[gated] {msg}", flush=True)


def check_close(y, y_ref, what, y_ungated=None):
    y = np.asarray(y, np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y - y_ref))
    assert np.all(np.isfinite(y)) and err <= TOL * rms, f"{what}: max|err| {err / rms:.2e} rms"
    if y_ungated is not None:   # the gate is in effect: the ungated output is far off
        assert np.max(np.abs(y - y_ungated)) > 20 * TOL * rms, what
    say(f"{what}: max|err| {err / rms:.2e} rms")


def check_route(r, ref, what):
    np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32),
                                  err_msg=f"{what} logits")
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"], err_msg=f"{what} top-k")
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), ref["offsets"], err_msg=f"{what} offsets")
    np.testing.assert_array_equal(r["perm"].cpu().numpy(), ref["perm"], err_msg=f"{what} perm")


def ungated(lay, x, idx, w, tokens=None):
    g = lay.shared_gate
    lay.shared_gate = None
    try:
        return oracle.layer_tokens(lay, x, idx, w, tokens)
    finally:
        lay.shared_gate = g


def test_qwen_layer_prefill_and_decode():
    wl = synth.WORKLOADS["qwen_decode"]
    lay = synth.workload_layer(wl)
    assert lay.shared_gate is not None
    T = 200
    x, _, _ = synth.gen_tokens(wl.dims, T, 71)
    dl = DeviceLayer(lay, max_tokens=T)
    xd = tokens_to_device(x)
    r = dl.route(xd)
    torch.cuda.synchronize()
    ref = oracle.route(lay, x)
    check_route(r, ref, "qwen T=200")
    y_ref = oracle.layer_tokens(lay, x, ref["idx"], ref["w"])
    y_ung = ungated(lay, x, ref["idx"], ref["w"])
    y = dl.prefill(xd)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref, "qwen prefill T=200", y_ung)
    for Td in (1, 5, 16):
        y = dl.decode(xd[:Td])
        torch.cuda.synchronize()
        check_close(y.cpu().numpy(), y_ref[:Td], f"qwen decode T={Td}", y_ung[:Td])
    dl.close()


def test_qwen_prefill_4096_all_tokens():
    wl = synth.WORKLOADS["qwen_prefill4096"]
    lay = synth.workload_layer(wl)
    x, tied, _ = synth.workload_tokens(wl, lay)
    T = wl.tokens
    dl = DeviceLayer(lay, max_tokens=T)
    xd = tokens_to_device(x)
    r = dl.route(xd)
    y = dl.prefill(xd)
    torch.cuda.synchronize()
    ref = oracle.route(lay, x)
    check_route(r, ref, "qwen T=4096")
    y_ref = np.empty((T, wl.dims.d_model), np.float64)
    for c in range(0, T, 1024):   # the oracle on every token, in chunks (progress lines)
        toks = np.arange(c, min(c + 1024, T), dtype=np.int32)
        y_ref[toks] = oracle.layer_tokens(lay, x, ref["idx"], ref["w"], toks)
        say(f"qwen T=4096 oracle tokens {c}..{toks[-1]}")
    sample = np.unique(np.concatenate([[0, T - 1], tied[:4], np.arange(0, T, 97)])).astype(np.int32)
    check_close(y.cpu().numpy(), y_ref, f"qwen prefill T=4096 (all tokens)")
    check_close(y.cpu().numpy()[sample], y_ref[sample], f"qwen prefill T=4096 gate in effect ({len(sample)} tokens)",
                ungated(lay, x, ref["idx"], ref["w"], sample))
    dl.close()


def test_gate_with_router_prologue():
    """The gate reads x, not the router prologue's output u."""
    dims = synth.Dims(d_model=512, n_experts=16, top_k=4, d_expert=128, d_shared=256)
    lay = synth.gen_layer(dims, 73, router="normal", shared_gate=True)
    rng = np.random.default_rng(73)
    lay.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, dims.d_model).astype(np.float32))
    x, _, _ = synth.gen_tokens(dims, 70, 73)
    dl = DeviceLayer(lay, max_tokens=70)
    xd = tokens_to_device(x)
    ref = oracle.route(lay, x)
    y_ref = oracle.layer_tokens(lay, x, ref["idx"], ref["w"])
    y_ung = ungated(lay, x, ref["idx"], ref["w"])
    y = dl.prefill(xd)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref, "prologue + gate prefill T=70", y_ung)
    y = dl.decode(xd[:3])
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref[:3], "prologue + gate decode T=3", y_ung[:3])
    dl.close()
