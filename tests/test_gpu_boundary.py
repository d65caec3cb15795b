"""GPU checks of the C-ABI boundary against the CPU oracle (MI355X only).

* Widths that are multiples of 64 but not of 128 (d_model 192, odd group counts along every
  projection).
* Expert scales far from the stated U(0.002, 0.02): around 1e-5 (below fp16's normal range)
  and above 2^-4, within one layer. The prefill GEMMs stage weights in fp16 with a per-matrix
  power-of-two exponent, so both paths stay within the output tolerance; metadata that cannot
  be staged (NaN scales, biases 2^24 times the largest scale) is refused at creation
  (Mference system design, ".gturbo directory": incompatible quantization metadata is
  rejected).
* MOE_FLAG_CHECK_FINITE: non-finite inputs are refused before anything is enqueued, a
  non-finite output is reported, finite calls give the same bits as without the flag
  (Mference, "Correctness and safety invariants": refuse rather than emit corrupt output).
  Inputs or hidden activations beyond fp16's range (the experts' operand type) make the
  output non-finite instead of clipping it, so the flag catches them too.
* Profiling on and off give bit-identical outputs (Gem native architecture, "Ownership
  boundaries": the profiled route must match the ordinary one).
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
    print(f"[boundary] {msg}", flush=True)


def check_close(y, ref, what, tol=TOL):
    y = np.asarray(y, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.max(np.abs(y - ref)) / rms
    assert np.all(np.isfinite(y)), what
    assert err <= tol, f"{what}: max|err| {err:.2e} rms"
    return err


def check_layer(lay, x, what, max_tokens=None):
    """Routing bit-exact, decode (in calls of at most 16 tokens) and prefill within tolerance."""
    T = x.shape[0]
    dl = DeviceLayer(lay, max_tokens or max(T, 16))
    xd = tokens_to_device(x)
    r = dl.route(xd)
    y_pre = dl.prefill(xd)
    y_dec = torch.empty_like(y_pre)
    for c in range(0, T, 16):
        dl.decode(xd[c:c + 16], y_dec[c:c + 16])
    torch.cuda.synchronize()
    ref, rr = oracle.layer_forward(lay, x)
    np.testing.assert_array_equal(r["logits"].cpu().numpy().view(np.uint32), rr["logits"].view(np.uint32))
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), rr["idx"])
    np.testing.assert_array_equal(r["perm"].cpu().numpy(), rr["perm"])
    e1 = check_close(y_pre.cpu().numpy(), ref, f"{what} prefill")
    e2 = check_close(y_dec.cpu().numpy(), ref, f"{what} decode")
    dl.close()
    say(f"{what}: routing exact, prefill {e1:.2e} rms, decode {e2:.2e} rms")


def test_d_model_multiple_of_64_not_128():
    D = synth.Dims(d_model=192, n_experts=16, top_k=4, d_expert=192, d_shared=320)
    lay = synth.gen_layer(D, 11, router="normal", zipf_s=0.7)
    x, _, _ = synth.gen_tokens(D, 140, 11)
    check_layer(lay, x, "d_model 192")


def _rescale(m: synth.QMat, rng, lo, hi, experts=None):
    """Redraw the scales of m (all matrices, or the listed experts) from U(lo, hi), with biases
    -8 * scale + N(0, 1e-3 * hi / 0.02) as the stated recipe scales them."""
    s = m.scales.copy()
    b = m.biases.copy()
    sel = slice(None) if experts is None else experts
    shape = s[sel].shape
    sv = rng.uniform(lo, hi, shape).astype(np.float32)
    s_bits = synth.f32_to_bf16_bits(sv)
    bv = -8.0 * synth.bf16_bits_to_f32(s_bits) + rng.standard_normal(shape).astype(np.float32) * np.float32(
        1e-3 * hi / 0.02)
    s[sel] = s_bits
    b[sel] = synth.f32_to_bf16_bits(bv)
    return synth.QMat(m.codes, s, b, m.bits, m.out_dim, m.in_dim)


def test_expert_scales_far_from_the_stated_range():
    """Scales around 1e-5 (whose fp16 value would be subnormal) for some experts and the shared
    expert, above 2^-4 for others: the prefill GEMMs' per-matrix staging exponent keeps 11
    significant bits either way."""
    D = synth.Dims(d_model=512, n_experts=16, top_k=4, d_expert=256, d_shared=256)
    lay = synth.gen_layer(D, 12, router="normal")
    rng = np.random.default_rng(12)
    small, large = np.arange(0, 16, 2), np.arange(1, 16, 4)
    for name in ("gate", "up", "down"):
        m = _rescale(getattr(lay, name), rng, 5e-6, 2e-5, experts=small)
        m = _rescale(m, rng, 0.1, 0.5, experts=large)
        setattr(lay, name, m)
    for name in ("sh_gate", "sh_up", "sh_down"):
        setattr(lay, name, _rescale(getattr(lay, name), rng, 5e-6, 2e-5))
    x, _, _ = synth.gen_tokens(D, 200, 12)
    check_layer(lay, x, "scales 5e-6..2e-5 and 0.1..0.5")


@pytest.mark.parametrize("bad", ["nan_scale", "inf_bias", "huge_bias"])
def test_create_refuses_unstageable_metadata(bad):
    D = synth.Dims(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256)
    lay = synth.gen_layer(D, 13, router="uniform")
    m = lay.down
    s, b = m.scales.copy(), m.biases.copy()
    if bad == "nan_scale":
        s[3, 7, 1] = 0x7FC0
    elif bad == "inf_bias":
        b[5, 0, 0] = 0xFF80
    else:   # |bias| 2^24 times the largest scale's power of two
        b[2, 9, 1] = synth.f32_to_bf16_bits(np.array([0.03 * 2 ** 25], np.float32))[0]
    lay.down = synth.QMat(m.codes, s, b, m.bits, m.out_dim, m.in_dim)
    with pytest.raises(B.MoeError) as ei:
        DeviceLayer(lay, 16)
    assert ei.value.status == B.MOE_E_QUANT
    say(f"create refuses {bad}: {ei.value}")


def test_check_finite_flag():
    w = synth.WORKLOADS["tiny"]
    lay = synth.workload_layer(w)
    x, _, _ = synth.gen_tokens(lay.dims, 40, 21)
    plain = DeviceLayer(lay, 64)
    chk = DeviceLayer(lay, 64, flags=B.MOE_FLAG_CHECK_FINITE)
    xd = tokens_to_device(x)
    for T in (40, 16):
        call = (lambda L, y: L.prefill(xd[:T], y)) if T > 16 else (lambda L, y: L.decode(xd[:T], y))
        ya = torch.empty((T, lay.dims.d_model), dtype=torch.float32, device="cuda:0")
        yb = torch.empty_like(ya)
        call(plain, ya)
        call(chk, yb)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int32), yb.view(torch.int32))
    # a NaN or an infinity in the input: refused, nothing written
    bad = x.copy()
    bad[3, 17] = 0x7FC0   # NaN
    bad[9, 5] = 0xFF80    # -inf
    bd = tokens_to_device(bad)
    for path, T in (("prefill", 40), ("decode", 16), ("route", 16)):
        y = torch.full((T, lay.dims.d_model), 7.0, device="cuda:0")
        with pytest.raises(B.MoeError) as ei:
            if path == "prefill":
                chk.prefill(bd[:T], y)
            elif path == "decode":
                chk.decode(bd[:T], y)
            else:
                chk.route(bd[:T])
        assert ei.value.status == B.MOE_E_NONFINITE
        torch.cuda.synchronize()
        assert torch.all(y == 7.0)
    # finite input whose router logits overflow: the non-finite output is reported
    big = synth.f32_to_bf16_bits(np.full((4, lay.dims.d_model), 3e38, np.float32))
    with pytest.raises(B.MoeError) as ei:
        chk.prefill(tokens_to_device(big))
    assert ei.value.status == B.MOE_E_NONFINITE and "output" in str(ei.value)
    # the handle stays usable
    y = chk.decode(xd[:4])
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), oracle.layer_forward(lay, x[:4])[0], "after refusals")
    plain.close()
    chk.close()
    say("check-finite flag: identical when finite, refuses NaN/inf inputs, reports non-finite outputs")


def test_values_beyond_fp16_range_make_the_output_nonfinite():
    """The experts read x and the hidden activation in fp16: a finite bf16 input above 65504, or
    a hidden activation above it (gate/up scales of 8), gives a non-finite output instead of a
    silently clipped one, and MOE_FLAG_CHECK_FINITE reports it for decode and prefill."""
    D = synth.Dims(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256)
    lay = synth.gen_layer(D, 14, router="uniform")
    x, _, _ = synth.gen_tokens(D, 24, 14)
    big_x = x.copy()
    big_x[5, 40] = synth.f32_to_bf16_bits(np.array([1.0e5], np.float32))[0]
    big_h = synth.gen_layer(D, 14, router="uniform")
    for name in ("gate", "up", "sh_gate", "sh_up"):
        setattr(big_h, name, _rescale(getattr(big_h, name), np.random.default_rng(15), 8.0, 8.0))
    for what, L, xx, row in (("x above 65504", lay, big_x, 5), ("hidden activation above 65504", big_h, x, None)):
        plain = DeviceLayer(L, 32)
        chk = DeviceLayer(L, 32, flags=B.MOE_FLAG_CHECK_FINITE)
        xd = tokens_to_device(xx)
        for path, T in (("prefill", 24), ("decode", 16)):
            y = plain.prefill(xd[:T]) if path == "prefill" else plain.decode(xd[:T])
            torch.cuda.synchronize()
            yn = y.cpu().numpy()
            if row is not None:
                assert not np.all(np.isfinite(yn[row])), f"{what} {path}"
                ok = np.ones(T, bool)
                ok[row] = False
                assert np.all(np.isfinite(yn[ok])), f"{what} {path}: other tokens stay finite"
            else:
                assert not np.all(np.isfinite(yn)), f"{what} {path}"
            with pytest.raises(B.MoeError) as ei:
                chk.prefill(xd[:T]) if path == "prefill" else chk.decode(xd[:T])
            assert ei.value.status == B.MOE_E_NONFINITE and "output" in str(ei.value)
        plain.close()
        chk.close()
        say(f"{what}: non-finite output, reported under the check-finite flag (decode and prefill)")


def test_x_beyond_fp16_range_is_infinite_on_both_paths():
    """Both paths convert x to fp16 rounding to nearest: with the gate/up weights of x's first
    input group made tiny (so x clipped to 65504 would still give finite hidden activations), an
    input of 1e5 in that group makes its token's output non-finite in decode as in prefill, while
    6e4 (below 65504) keeps every output finite."""
    D = synth.Dims(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256)
    lay = synth.gen_layer(D, 16, router="uniform")
    for name in ("gate", "up", "sh_gate", "sh_up"):
        m = getattr(lay, name)
        sc, bi = m.scales.copy(), m.biases.copy()
        sc[..., 0] = synth.f32_to_bf16_bits(np.full(sc[..., 0].shape, 1e-7, np.float32))
        bi[..., 0] = synth.f32_to_bf16_bits(np.full(bi[..., 0].shape, -4e-7, np.float32))
        setattr(lay, name, synth.QMat(m.codes, sc, bi, m.bits, m.out_dim, m.in_dim))
    x, _, _ = synth.gen_tokens(D, 16, 16)
    dl = DeviceLayer(lay, 16)
    for v, finite in ((1.0e5, False), (6.0e4, True)):
        xx = x.copy()
        xx[5, 40] = synth.f32_to_bf16_bits(np.array([v], np.float32))[0]
        xd = tokens_to_device(xx)
        for path in ("prefill", "decode"):
            y = (dl.prefill(xd) if path == "prefill" else dl.decode(xd)).cpu().numpy()
            assert np.all(np.isfinite(np.delete(y, 5, axis=0))), f"x = {v:g} {path}: other tokens"
            assert bool(np.all(np.isfinite(y[5]))) == finite, f"x = {v:g} {path}"
    dl.close()
    say("x = 1e5 (tiny weights on its group): non-finite output in decode and prefill; x = 6e4: finite")


def test_profiling_does_not_change_results():
    wd = synth.WORKLOADS["prefill512"]
    lay = synth.workload_layer(wd)
    x, _, _ = synth.workload_tokens(wd, lay)
    dl = DeviceLayer(lay, 512)
    xd = tokens_to_device(x)
    outs = {}
    for on in (False, True, False):
        B.moe_profile_enable(dl.handle, on)
        yp = dl.prefill(xd)
        yd = dl.decode(xd[:16])
        torch.cuda.synchronize()
        outs.setdefault(on, []).append((yp.view(torch.int32).clone(), yd.view(torch.int32).clone()))
    ref = outs[False][0]
    for yp, yd in outs[True] + outs[False][1:]:
        assert torch.equal(yp, ref[0]) and torch.equal(yd, ref[1])
    ms, n = B.moe_profile_read(dl.handle, B.kernel_id("pre_gateup"))
    assert n == 1 and ms > 0
    dl.close()
    say("profiling on and off: prefill and decode outputs bit-identical")


def test_last_routing_errors():
    lay = synth.workload_layer(synth.WORKLOADS["tiny"])
    dl = DeviceLayer(lay, 16)
    idx = torch.empty((16, 2), dtype=torch.int32, device="cuda:0")
    w = torch.empty((16, 2), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as ei:
        B.moe_last_routing(dl.handle, 1, idx, w)   # nothing has run
    assert ei.value.status == B.MOE_E_INVALID
    x, _, _ = synth.gen_tokens(lay.dims, 4, 3)
    dl.decode(tokens_to_device(x))
    with pytest.raises(B.MoeError) as ei:
        B.moe_last_routing(dl.handle, 5, idx, w)   # more tokens than the call had
    assert ei.value.status == B.MOE_E_INVALID
    B.moe_last_routing(dl.handle, 4, idx, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx[:4].cpu().numpy(), oracle.route(lay, x)["idx"])
    dl.close()
