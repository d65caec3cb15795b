"""moe_forward_decode_noalloc: the handle-free decode that allocates nothing (its scratch is
one static device array per device) must give the same bits as moe_forward_decode on the
same layer, call after call, whatever the previous call left in the shared array."""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import binding as B
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[noalloc] {msg}", flush=True)


def _pair(dl, x, T):
    """(moe_forward_decode output, moe_forward_decode_noalloc output) for the first T tokens."""
    xd = tokens_to_device(x[:T])
    y_ref = torch.empty((T, dl.dims_py.d_model), dtype=torch.float32, device="cuda:0")
    y = torch.full_like(y_ref, float("nan"))
    B.moe_forward_decode(dl.handle, xd, T, y_ref)
    B.moe_forward_decode_noalloc(dl.dims, dl.weights, xd, T, y)
    torch.cuda.synchronize()
    return y_ref, y


@pytest.mark.parametrize("variant", ["plain", "prologue_gate"])
def test_noalloc_decode_matches_the_layer_handle(variant):
    w = synth.WORKLOADS["decode"]
    lay = synth.workload_layer(w)
    if variant == "prologue_gate":   # router prologue, per-expert scale and a gated shared expert
        rng = np.random.default_rng(31)
        D = lay.dims
        lay.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D.d_model).astype(np.float32))
        lay.per_expert_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, D.n_experts).astype(np.float32))
        lay.shared_gate = synth.f32_to_bf16_bits(rng.normal(0.0, D.d_model ** -0.5, D.d_model).astype(np.float32))
    x, _, _ = synth.gen_tokens(lay.dims, 16, 77)
    dl = DeviceLayer(lay, max_tokens=16)
    for T in (16, 5, 1):   # each call after a larger one: the shared array holds the previous call's values
        y_ref, y = _pair(dl, x, T)
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"T={T}"
        ref, _ = oracle.layer_forward(lay, x[:T])
        got = y.cpu().numpy().astype(np.float64)
        err = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
        assert err <= 2e-3, f"T={T}: max|err| {err:.2e} rms"
        say(f"{variant} T={T}: bit-identical to the handle path, oracle max|err| {err:.2e} rms")
    dl.close()


def test_noalloc_refuses_what_it_cannot_hold():
    lay = synth.workload_layer(synth.WORKLOADS["tiny"])
    dl = DeviceLayer(lay, max_tokens=8)
    x = tokens_to_device(synth.gen_tokens(lay.dims, 16, 3)[0])
    y = torch.empty((16, lay.dims.d_model), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as ei:   # above the layer's max_tokens
        B.moe_forward_decode_noalloc(dl.dims, dl.weights, x, 9, y)
    assert ei.value.status == B.MOE_E_CAPACITY
    y_ref, y2 = _pair(dl, synth.gen_tokens(lay.dims, 8, 4)[0], 8)   # still usable
    assert torch.equal(y2.view(torch.int32), y_ref.view(torch.int32))
    dl.close()
