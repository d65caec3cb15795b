"""GPU parity of the 30-layer decode stack (2816-wide layers, distinct seeded weights per
layer, 256 consecutive tokens, residual stream between layers), through the C ABI.

Every layer is checked against the CPU oracle on the GPU's own input to that layer (teacher
forcing) for all 256 tokens, run as 16-token decode calls: router top-k sets bit-exact (the
decode launch's own selection, read back through moe_last_routing), layer output within
max |err| <= 2e-3 * rms, and the residual step (h + y, then the norm) bit-exact, both sides
rounding the fp64 value once to bf16. The whole stack then runs one token at a time through
moe_stack_forward_decode, and its final residual stream must equal, bit for bit, the
layer-by-layer run on every token (decode results do not depend on how many tokens share a
call).
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
CALL = 16   # tokens per decode call (the decode path's capacity)


def say(msg):
    print(f"[stack] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def test_stack_30_layers_256_tokens():
    w = synth.WORKLOADS["stack"]
    D = w.dims
    T, NL, k = w.tokens, w.layers, w.dims.top_k
    h0 = synth.gen_stack_tokens(D, T, w.seed)
    dev = torch.device("cuda:0")

    hs = tokens_to_device(h0, dev)
    xs = torch.empty_like(hs)
    ys = torch.empty((T, D.d_model), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    B.moe_stack_glue(hs, None, hs, xs, T, D.d_model)
    torch.cuda.synchronize()
    hn_ref, xn_ref = oracle.stack_glue(h0, None)
    np.testing.assert_array_equal(bits(hs), hn_ref)
    np.testing.assert_array_equal(bits(xs), xn_ref)

    layers = []
    worst = 0.0
    for l in range(NL):
        lay = synth.workload_layer(w, l)
        dl = DeviceLayer(lay, max_tokens=CALL, device=dev)
        layers.append(dl)
        x_l = bits(xs)
        for c in range(0, T, CALL):
            dl.decode(xs[c:c + CALL], ys[c:c + CALL])
            B.moe_last_routing(dl.handle, CALL, idx[c:c + CALL], wts[c:c + CALL])
        h_prev = bits(hs)
        B.moe_stack_glue(hs, ys, hs, xs, T, D.d_model)
        torch.cuda.synchronize()
        ref_r = oracle.route(lay, x_l)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_r["idx"], err_msg=f"layer {l} decode top-k")
        np.testing.assert_allclose(wts.cpu().numpy(), ref_r["w"], rtol=2e-6, atol=1e-7,
                                   err_msg=f"layer {l} decode routing weights")
        y_ref = oracle.layer_tokens(lay, x_l, ref_r["idx"], ref_r["w"])
        y_gpu = ys.cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(y_ref ** 2))
        err = np.max(np.abs(y_gpu - y_ref)) / rms
        worst = max(worst, err)
        assert err <= TOL, f"layer {l}: max|err| {err:.2e} rms"
        hn_ref, xn_ref = oracle.stack_glue(h_prev, y_gpu)
        np.testing.assert_array_equal(bits(hs), hn_ref, err_msg=f"layer {l} residual")
        np.testing.assert_array_equal(bits(xs), xn_ref, err_msg=f"layer {l} norm")
        say(f"layer {l}: {T} tokens, top-k exact, max|err| {err:.2e} rms, residual and norm bit-exact")
        del lay
    say(f"worst layer error {worst:.2e} rms")

    # the whole stack, one token at a time, through the stack entry point
    h = tokens_to_device(h0, dev)
    xb = torch.empty((1, D.d_model), dtype=torch.int16, device=dev)
    yb = torch.empty((1, D.d_model), dtype=torch.float32, device=dev)
    hb = torch.empty_like(xb)
    handles = [L.handle for L in layers]
    for t in range(T):
        B.moe_stack_forward_decode(handles, h[t:t + 1], 1, xb, yb, hb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(h), bits(hs))
    say(f"stack entry point: {T} tokens x {NL} layers one at a time, every row identical to the "
        f"layer-by-layer run")
    # 16 tokens per call: the residual step runs in its own launch (T d above the router's LDS
    # budget) and gives the same bits
    hS = tokens_to_device(h0[:CALL], dev)
    xS, hbS = torch.empty_like(hS), torch.empty_like(hS)
    yS = torch.empty((CALL, D.d_model), dtype=torch.float32, device=dev)
    B.moe_stack_forward_decode(handles, hS, CALL, xS, yS, hbS)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(hS), bits(hs)[:CALL])
    say(f"stack entry point with {CALL} tokens per call: identical")
    for L in layers:
        L.close()


def test_stack_rejects_mixed_widths_and_capacity():
    tiny = synth.workload_layer(synth.WORKLOADS["tiny"])
    narrow = synth.gen_layer(synth.Dims(d_model=128, n_experts=8, top_k=2, d_expert=64, d_shared=64), 5,
                             router="uniform")
    a = DeviceLayer(tiny, max_tokens=4)
    b = DeviceLayer(narrow, max_tokens=4)
    h = torch.zeros((8, tiny.dims.d_model), dtype=torch.int16, device="cuda:0")
    xb = torch.empty_like(h)
    yb = torch.empty((8, tiny.dims.d_model), dtype=torch.float32, device="cuda:0")
    hb = torch.empty_like(h)
    with pytest.raises(B.MoeError) as ei:
        B.moe_stack_forward_decode([a.handle, a.handle], h, 8, xb, yb, hb)
    assert ei.value.status == B.MOE_E_CAPACITY
    with pytest.raises(B.MoeError) as ei:
        B.moe_stack_forward_decode([a.handle, b.handle], h, 1, xb, yb, hb)
    assert ei.value.status == B.MOE_E_SHAPE
    h0 = h.clone()
    B.moe_stack_forward_decode([a.handle, a.handle], h, 0, xb, yb, hb)     # T = 0: no-op
    torch.cuda.synchronize()
    assert torch.equal(h, h0)
    a.close()
    b.close()


def test_stack_plan_replays_match_the_direct_call():
    """moe_stack_plan_create records the stack call once; every replay on the same buffers gives,
    bit for bit, the direct call's h, x_buf and y_buf, with other work on the same layers (direct
    calls on other buffers) and host copies of the next token's stream between the replays."""
    w = synth.WORKLOADS["stack"]
    D = w.dims
    NL = 6
    dev = torch.device("cuda:0")
    layers = [DeviceLayer(synth.workload_layer(w, l), max_tokens=CALL, device=dev) for l in range(NL)]
    handles = [L.handle for L in layers]
    h0 = tokens_to_device(synth.gen_stack_tokens(D, 40, w.seed + 7), dev)
    for T in (1, 4):
        h = torch.empty((T, D.d_model), dtype=torch.int16, device=dev)
        xb, hb = torch.empty_like(h), torch.empty_like(h)
        yb = torch.empty((T, D.d_model), dtype=torch.float32, device=dev)
        h2, xb2, hb2 = torch.empty_like(h), torch.empty_like(h), torch.empty_like(h)
        yb2 = torch.empty_like(yb)
        plan = B.moe_stack_plan_create(handles, h, T, xb, yb, hb)
        try:
            for step in range(8):
                toks = h0[T * step: T * step + T]
                h2.copy_(toks)
                B.moe_stack_forward_decode(handles, h2, T, xb2, yb2, hb2)   # the direct call
                h.copy_(toks)
                B.moe_stack_plan_run(plan)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(bits(h), bits(h2))
                np.testing.assert_array_equal(bits(xb), bits(xb2))
                np.testing.assert_array_equal(yb.cpu().numpy().view(np.uint32), yb2.cpu().numpy().view(np.uint32))
        finally:
            B.moe_stack_plan_destroy(plan)
        say(f"stack plan, {NL} layers, T={T}: 8 replays bit-identical to the direct call")
    # calls that read device memory back cannot be recorded
    B.moe_profile_enable(handles[2], True)
    with pytest.raises(B.MoeError) as ei:
        B.moe_stack_plan_create(handles, h, 1, xb, yb, hb)
    assert ei.value.status == B.MOE_E_INVALID
    B.moe_profile_enable(handles[2], False)
    with pytest.raises(B.MoeError) as ei:
        B.moe_stack_plan_create(handles, h, CALL + 1, xb, yb, hb)
    assert ei.value.status == B.MOE_E_CAPACITY
    for L in layers:
        L.close()
