"""GPU parity in the integer-exact regime, through the C ABI: a layer whose every intermediate
value is exactly representable, so the GPU's fp32 outputs must equal the oracle's float64 ones
bit for bit, in decode and in prefill (the GEMVs and the GEMMs alike).

* Inputs are bf16 values in {-2, 0, 2}.
* Every expert matrix has scale 1 and bias -8 in every group, so a weight is its code minus 8
  (the affine definition, Mference system design, "Why the runtime has this shape"); the same
  weights also run as Q4_0 experts with d = 1.
* Each gate row and each up row has one code other than 8, so it reads one input: g is 0, +-14
  or +-16. There GELU-tanh is exactly g (tanh rounds to 1) or a signed zero (tanh rounds to -1),
  in fp32 and in float64. u is an even integer of magnitude at most 16, and h = gelu(g) u is an
  integer of magnitude at most 256, which is exact in fp16.
* Down rows have random codes, so r and the shared output are integers below 2^19.
* The router's experts come in identical pairs (rows 2i and 2i + 1 equal). Every token's top-2
  is then a tied pair, with routing weights exactly 1/2, and y = sh + r_a / 2 + r_b / 2 is a
  multiple of 1/2.

A dropped term, a wrong row or group, or a wrong scale shows up as a difference in the bits,
not as a tolerance question.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

BF16_ONE, BF16_MINUS8 = 0x3F80, 0xC100
BF16_TWO, BF16_MINUS2 = 0x4000, 0xC000


def say(msg):
    print(f"[exact] {msg}", flush=True)


def one_input_rows(m, rng, codes_for_input):
    """Codes 8 (weight 0) everywhere except one random input per row, which gets a code drawn
    from codes_for_input."""
    full = np.full(m.codes.shape[:-1] + (m.in_dim,), 8, np.uint8)
    rows = full.reshape(-1, m.in_dim)
    j = rng.integers(m.in_dim, size=rows.shape[0])
    rows[np.arange(rows.shape[0]), j] = rng.choice(codes_for_input, size=rows.shape[0])
    m.codes[...] = full[..., 0::2] | (full[..., 1::2] << 4)


def as_q4_0(lay):
    """The same weights as Q4_0 experts: blocks of 32 codes with d = 1, weight d (q - 8) (Gem
    native architecture, "M4 Max operating assumptions"), byte j of a block holding element j in
    its low and element j + 16 in its high nibble."""
    qd = synth.Dims(d_model=lay.dims.d_model, n_experts=lay.dims.n_experts, top_k=lay.dims.top_k,
                    d_expert=lay.dims.d_expert, d_shared=lay.dims.d_shared, expert_format="q4_0")
    qlay = synth.gen_layer(qd, 61)
    qlay.router = lay.router
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        m = getattr(lay, name)
        q = np.stack([m.codes & 0x0F, m.codes >> 4], axis=-1).reshape(m.codes.shape[:-1] + (m.in_dim,))
        qb = q.reshape(q.shape[:-1] + (m.in_dim // 32, 32))
        blk = np.empty(qb.shape[:-1] + (18,), np.uint8)
        blk[..., :2] = np.full(qb.shape[:-1] + (1,), 1.0, np.float16).view(np.uint8)
        blk[..., 2:] = (qb[..., :16] | (qb[..., 16:] << 4)).astype(np.uint8)
        getattr(qlay, name).codes = blk.reshape(getattr(qlay, name).codes.shape)
    return qlay


def exact_layer():
    dims = synth.Dims(d_model=512, n_experts=8, top_k=2, d_expert=128, d_shared=192)
    lay = synth.gen_layer(dims, 61)
    rng = np.random.default_rng(62)
    for m in (lay.gate, lay.up, lay.down, lay.sh_gate, lay.sh_up, lay.sh_down):
        m.scales[...] = BF16_ONE
        m.biases[...] = BF16_MINUS8
    for m in (lay.gate, lay.sh_gate):     # weight 7 or -8 on one input: g in {0, +-14, +-16}
        one_input_rows(m, rng, np.array([15, 0], np.uint8))
    for m in (lay.up, lay.sh_up):         # weight -8..7 on one input: u in {0, +-2w}
        one_input_rows(m, rng, np.arange(16, dtype=np.uint8))
    r = lay.router
    r.codes[1::2] = r.codes[0::2]
    r.scales[1::2] = r.scales[0::2]
    r.biases[1::2] = r.biases[0::2]
    return lay


def exact_tokens(dims, T, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(np.array([BF16_MINUS2, 0, BF16_TWO], np.uint16), size=(T, dims.d_model))


def check_exact(y_gpu, y_ref, what):
    y_gpu = np.asarray(y_gpu)
    assert y_gpu.dtype == np.float32
    bad = np.nonzero(y_gpu.astype(np.float64) != y_ref)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} of {y_ref.size} outputs differ, first at "
                              f"{bad[0][0], bad[1][0]}: {y_gpu[bad[0][0], bad[1][0]]!r} vs {y_ref[bad[0][0], bad[1][0]]!r}")
    say(f"{what}: all {y_ref.size} outputs equal the oracle's (max |y| {np.max(np.abs(y_ref)):.0f})")


@pytest.mark.parametrize("fmt", ["affine", "q4_0"])
def test_integer_exact_layer_is_bit_identical_in_decode_and_prefill(fmt):
    lay = exact_layer()
    if fmt == "q4_0":
        lay = as_q4_0(lay)
    T = 300
    x = exact_tokens(lay.dims, T, 63)
    ref = oracle.route(lay, x)
    # the regime: tied pairs with weights exactly 1/2, and every output a multiple of 1/2 that
    # fp32 holds exactly (so exact arithmetic on both sides must give the same bits)
    assert np.all(ref["idx"][:, 0] % 2 == 0) and np.all(ref["idx"][:, 1] == ref["idx"][:, 0] + 1)
    assert np.all(ref["w"] == 0.5)
    y_ref = oracle.layer_tokens(lay, x, ref["idx"], ref["w"])
    assert np.all(2 * y_ref == np.round(2 * y_ref)) and np.max(np.abs(y_ref)) < 2 ** 22
    assert np.count_nonzero(y_ref) > 0.9 * y_ref.size

    dl = DeviceLayer(lay, max_tokens=T)
    xd = tokens_to_device(x)
    say(f"route T={T}")
    r = dl.route(xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), ref["idx"])
    assert np.all(r["w"].cpu().numpy() == 0.5)
    np.testing.assert_array_equal(r["perm"].cpu().numpy(), ref["perm"])
    for n in (T, 129, 1):
        say(f"prefill T={n}")
        y = dl.prefill(xd[:n])
        torch.cuda.synchronize()
        check_exact(y.cpu().numpy(), y_ref[:n], f"{fmt} prefill T={n}")
    for n in (1, 5, 16):
        say(f"decode T={n}")
        y = dl.decode(xd[:n])
        torch.cuda.synchronize()
        check_exact(y.cpu().numpy(), y_ref[:n], f"{fmt} decode T={n}")
    dl.close()
