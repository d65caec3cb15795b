"""GPU parity of Q4_0 expert matrices (MOE_FORMAT_Q4_0) against the CPU oracle, through the C ABI.

Q4_0 (Gem native architecture, "M4 Max operating assumptions": 32 weights in an 18-byte block;
"Ownership boundaries": the GGUF loader accepts Q4_0 matrices) stores weight d (code - 8) with
one fp16 d per 32 inputs. The decode kernels split each 64-input group into its two blocks;
the prefill GEMMs stage fp16(2^m (d q - 8 d)) with the K-steps of each block taking its d.

* Routing bit-exact, decode and prefill within max |err| <= 2e-3 rms of the oracle on every
  token: a small layer with ragged tiles, the 2816-wide layer (512-token chunk, decode at 1 and
  16 tokens), and a layer with fp16-subnormal block scales in some experts and scales near 2^-4
  in others.
* A Q4_0 layer whose two blocks per group share d equals the affine layer with scale d and bias
  -8 d: the prefill GEMMs then stage the same fp16 weights, so the two layers' prefill outputs
  are bit-identical (decode rounds its per-block sums differently and is checked against the
  oracle).
* Expert slots and the handle-free decode run Q4_0 layers with the bits of the resident layer.
* A NaN or infinite d is refused at creation (MOE_E_QUANT).
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


def say(msg):
    print(f"[q4_0] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y))
    return np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2))


def check_layer(lay, x, what, dec_chunk=16):
    T = x.shape[0]
    dl = DeviceLayer(lay, max(T, 16))
    xd = tokens_to_device(x)
    r = dl.route(xd)
    y_pre = dl.prefill(xd)
    y_dec = torch.empty_like(y_pre)
    for c in range(0, T, dec_chunk):
        dl.decode(xd[c:c + dec_chunk], y_dec[c:c + dec_chunk])
    torch.cuda.synchronize()
    ref, rr = oracle.layer_forward(lay, x)
    np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), rr["logits"].view(np.uint32))
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), rr["idx"])
    e1, e2 = rel_err(y_pre.cpu().numpy(), ref), rel_err(y_dec.cpu().numpy(), ref)
    assert e1 <= TOL, f"{what} prefill: {e1:.2e}"
    assert e2 <= TOL, f"{what} decode: {e2:.2e}"
    say(f"{what}: routing exact, prefill {e1:.2e} rms, decode {e2:.2e} rms")
    return dl


def test_small_layer_ragged_tiles():
    D = synth.Dims(d_model=320, n_experts=12, top_k=3, d_expert=192, d_shared=320, expert_format="q4_0")
    lay = synth.gen_layer(D, 41, router="normal", zipf_s=0.6)
    x, _, _ = synth.gen_tokens(D, 277, 41)
    check_layer(lay, x, "d 320, 12 experts, 277 tokens").close()


def test_full_width_layer_prefill_chunk_and_decode():
    w = synth.WORKLOADS["q4_0_prefill512"]
    lay = synth.workload_layer(w)
    x, _, _ = synth.workload_tokens(w, lay)
    dl = check_layer(lay, x, "2816-wide layer, 512 tokens")
    xd = tokens_to_device(x)
    ref1, _ = oracle.layer_forward(lay, x[:1])
    y1 = dl.decode(xd[:1])
    torch.cuda.synchronize()
    e = rel_err(y1.cpu().numpy(), ref1)
    assert e <= TOL
    say(f"2816-wide layer, decode T=1: {e:.2e} rms")
    dl.close()


def test_block_scales_across_fp16_range():
    """Experts whose block scales are fp16 subnormals (|d| in [2^-20, 2^-18]) and experts with
    |d| in [2^-5, 2^-3], in the same layer (each matrix's d within a factor of 4, as the affine
    boundary test varies scales per matrix): the prefill staging exponent follows each matrix's
    largest |d|, decode converts d exactly."""
    D = synth.Dims(d_model=512, n_experts=16, top_k=4, d_expert=256, d_shared=256, expert_format="q4_0")
    lay = synth.gen_layer(D, 43, router="normal")
    rng = np.random.default_rng(43)

    def redraw(m, lo, hi, experts=None):
        blk = m.codes.reshape(m.codes.shape[:-1] + (m.in_dim // 32, 18)).copy()
        sel = (slice(None),) if experts is None else (experts,)
        shape = blk[sel][..., 0].shape
        d = (np.exp2(rng.uniform(lo, hi, shape)) * np.where(rng.random(shape) < 0.5, -1, 1)).astype(np.float16)
        sub = blk[sel]
        sub[..., :2] = d[..., None].view(np.uint8)
        blk[sel] = sub
        m.codes = blk.reshape(m.codes.shape)

    small, large = np.arange(0, 16, 2), np.arange(1, 16, 4)
    for name in ("gate", "up", "down"):
        redraw(getattr(lay, name), -20, -18, small)
        redraw(getattr(lay, name), -5, -3, large)
    for name in ("sh_gate", "sh_up", "sh_down"):
        redraw(getattr(lay, name), -20, -18)
    assert np.any((lay.gate.codes.reshape(16, 256, 16, 18)[small, ..., 1] & 0x7C) == 0)   # subnormal d present
    x, _, _ = synth.gen_tokens(D, 150, 43)
    check_layer(lay, x, "block scales 2^-20..2^-18 and 2^-5..2^-3").close()


def test_equal_blocks_match_the_affine_layer_bit_for_bit_in_prefill():
    D = synth.Dims(d_model=768, n_experts=16, top_k=4, d_expert=320, d_shared=448)
    lay = synth.gen_layer(D, 45, router="normal", zipf_s=0.8)
    QD = synth.Dims(d_model=768, n_experts=16, top_k=4, d_expert=320, d_shared=448, expert_format="q4_0")
    qlay = synth.gen_layer(QD, 45, router="normal", zipf_s=0.8)
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        m = getattr(lay, name)
        sval = synth.bf16_bits_to_f32(m.scales)
        m.biases = synth.f32_to_bf16_bits(np.float32(-8.0) * sval)
        q = np.stack([m.codes & 0x0F, m.codes >> 4], axis=-1).reshape(m.codes.shape[:-1] + (m.in_dim,))
        qb = q.reshape(q.shape[:-1] + (m.in_dim // 32, 32))
        d16 = sval.astype(np.float16).repeat(2, axis=-1)
        blk = np.empty(qb.shape[:-1] + (18,), np.uint8)
        blk[..., :2] = d16[..., None].view(np.uint8)
        blk[..., 2:] = (qb[..., :16] | (qb[..., 16:] << 4)).astype(np.uint8)
        getattr(qlay, name).codes = blk.reshape(getattr(qlay, name).codes.shape)
    x, _, _ = synth.gen_tokens(D, 300, 45)
    xd = tokens_to_device(x)
    a = DeviceLayer(lay, 300)
    q = DeviceLayer(qlay, 300)
    ya, yq = a.prefill(xd), q.prefill(xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(yq), bits(ya))
    ref, _ = oracle.layer_forward(qlay, x[:16])
    yd = q.decode(xd[:16])
    torch.cuda.synchronize()
    e = rel_err(yd.cpu().numpy(), ref)
    assert e <= TOL
    say(f"equal blocks: prefill bit-identical to the affine layer (300 tokens), decode {e:.2e} rms")
    a.close()
    q.close()


def test_slots_and_noalloc_decode():
    D = synth.Dims(d_model=1024, n_experts=32, top_k=4, d_expert=256, d_shared=512, expert_format="q4_0")
    lay = synth.gen_layer(D, 47, router="normal", zipf_s=0.5)
    x, _, _ = synth.gen_tokens(D, 150, 47)
    xd = tokens_to_device(x)
    ref = DeviceLayer(lay, max_tokens=150)
    sl = DeviceLayer(lay, max_tokens=150, n_slots=8)
    y_ref = ref.prefill(xd)
    y, tiles, fills = sl.prefill_tiled(xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    assert B.moe_slot_faults(sl.handle) == 0
    e = rel_err(y.cpu().numpy(), oracle.layer_forward(lay, x)[0])
    assert e <= TOL
    sl.ensure(sl.route(xd[:2])["idx"].cpu().numpy().ravel())   # two tokens: at most 8 experts
    yd = sl.decode(xd[:2])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(yd), bits(ref.decode(xd[:2])))
    say(f"slots: 150 tokens in {tiles} expert tiles bit-identical to the resident layer ({e:.2e} rms); decode too")
    for T in (16, 3):
        y_h = torch.empty((T, D.d_model), dtype=torch.float32, device="cuda:0")
        y_n = torch.full_like(y_h, float("nan"))
        B.moe_forward_decode(ref.handle, xd[:T], T, y_h)
        B.moe_forward_decode_noalloc(ref.dims, ref.weights, xd[:T], T, y_n)
        torch.cuda.synchronize()
        assert torch.equal(y_n.view(torch.int32), y_h.view(torch.int32)), f"T={T}"
    say("handle-free decode: bit-identical to the handle path at T=16, 3")
    ref.close()
    sl.close()


@pytest.mark.parametrize("bad", [0x7E00, 0x7C00, 0xFC00])
def test_create_refuses_nonfinite_block_scales(bad):
    D = synth.Dims(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256, expert_format="q4_0")
    lay = synth.gen_layer(D, 49, router="uniform")
    blk = lay.up.codes.reshape(8, 128, 8, 18).copy()
    blk[5, 17, 3, :2] = np.array([bad & 0xFF, bad >> 8], np.uint8)
    lay.up.codes = blk.reshape(lay.up.codes.shape)
    with pytest.raises(B.MoeError) as ei:
        DeviceLayer(lay, 16)
    assert ei.value.status == B.MOE_E_QUANT
    say(f"create refuses d = {bad:#06x}")
