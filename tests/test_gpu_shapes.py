"""GPU parity on layer shapes away from the 2816-wide workload, through the C ABI: the
widest model dimension the kernels take (8192: router lanes loop over 128 groups), many
experts with the largest top-k (256 experts, top-16: four logits per lane in the top-k,
every down-projection wave shared), the largest expert count (1024, top-8), top-1 (a single routing weight of exactly 1), widths
whose last prefill tile is only partly filled, expert scales above 2^-4, and a chunk routed on
the matrix cores with ragged token, expert and group counts.
Each shape runs with affine group-64 experts and (except the rescaled-scale case, which is about
affine metadata) with Q4_0 experts. Same bar as the other parity tests: top-k index sets and
grouping bit-exact, outputs within max |err| <= 2e-3 * rms of the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

TOL = 2e-3

SHAPES = {
    "wide_d8192": (synth.Dims(d_model=8192, n_experts=16, top_k=4, d_expert=128, d_shared=128), 2, 130),
    "e256_top16": (synth.Dims(d_model=1024, n_experts=256, top_k=16, d_expert=256, d_shared=512), 3, 200),
    "top1": (synth.Dims(d_model=256, n_experts=4, top_k=1, d_expert=64, d_shared=64), 5, 70),
    # widths that leave the last prefill tile part-empty: 10 column blocks of 64 for the down
    # projection (tiles of 4), 6 and 10 hidden blocks of 32 for gate/up
    "ragged_tiles": (synth.Dims(d_model=640, n_experts=8, top_k=2, d_expert=192, d_shared=320), 3, 150),
    # expert scales and biases 8x the usual (scales up to 0.16): the prefill GEMMs must take the
    # dequantization that does not rely on scales below 2^-4
    "large_scales": (synth.Dims(d_model=512, n_experts=8, top_k=2, d_expert=128, d_shared=192), 2, 140),
    # the largest expert count the library takes (sixteen logits per lane in the top-k)
    "e1024_top8": (synth.Dims(d_model=512, n_experts=1024, top_k=8, d_expert=64, d_shared=128), 4, 260),
    # a chunk large enough for the matrix-core prefill router (32 x 18 router workgroups of the
    # group-split kernel would exceed its limit), with its last 64-token tile a quarter full, the
    # last 16-expert block half past the expert count, and an odd group count (9: three K steps of
    # four groups, the last holding a single group)
    "router_matrix_cores": (synth.Dims(d_model=576, n_experts=72, top_k=8, d_expert=128, d_shared=256), 2, 2000),
}


def times8(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns multiplied by 8 (exponent + 3; zeros stay zero)."""
    b = bits.astype(np.uint32)
    return np.where((b & 0x7FFF) != 0, b + (3 << 7), b).astype(np.uint16)


def check_close(y_gpu, y_ref, what):
    y_gpu = np.asarray(y_gpu, np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    err = np.max(np.abs(y_gpu - y_ref))
    assert np.all(np.isfinite(y_gpu)), what
    assert err <= TOL * rms, f"{what}: max|err| {err:.3e} > {TOL} * rms {rms:.3e}"
    print(f"[shapes] {what}: max|err| {err / rms:.2e} rms", flush=True)


# every shape with affine experts; the ones that do not rescale affine metadata with Q4_0 experts too
CASES = [(n, "affine") for n in SHAPES] + [(n, "q4_0") for n in SHAPES if n != "large_scales"]


@pytest.mark.parametrize("name,fmt", CASES)
def test_shape(name, fmt):
    dims, t_dec, t_pre = SHAPES[name]
    dims = dataclasses.replace(dims, expert_format=fmt)
    name = name if fmt == "affine" else f"{name} q4_0"
    lay = synth.gen_layer(dims, 11)
    if name == "large_scales":   # affine only
        for m in (lay.gate, lay.up, lay.down, lay.sh_gate, lay.sh_up, lay.sh_down):
            m.scales[...] = times8(m.scales)
            m.biases[...] = times8(m.biases)
        assert max(synth.bf16_bits_to_f32(m.scales).max() for m in (lay.gate, lay.down)) > 0.0625
    x, _, _ = synth.gen_tokens(dims, t_pre, 12)
    dl = DeviceLayer(lay, max_tokens=t_pre)
    xd = tokens_to_device(x)
    # routing and grouping, prefill-sized
    r = dl.route(xd)
    torch.cuda.synchronize()
    ref = oracle.route(lay, x)
    np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(r["perm"].cpu().numpy(), ref["perm"])
    if dims.top_k == 1:
        assert np.all(r["w"].cpu().numpy() == 1.0)
    y_ref = oracle.layer_tokens(lay, x, ref["idx"], ref["w"])
    y = dl.prefill(xd)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref, f"{name} prefill T={t_pre}")
    y = dl.decode(xd[:t_dec])
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), y_ref[:t_dec], f"{name} decode T={t_dec}")
    dl.close()
