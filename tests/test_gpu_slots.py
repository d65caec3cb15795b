"""GPU parity of the expert slot cache (Mference system design, "Load and ownership" and
"Decode": per-layer expert slots, LFU planning, a GPU-visible expert-to-slot table and a GPU
lookup of the selected experts), through the C ABI.

Every slot-path output is checked against the CPU oracle (max |err| <= 2e-3 * rms, top-k sets
bit-exact), and must also give the same bits as the same layer with every expert resident:
the kernels run the same arithmetic on the same weights, only their addresses differ. Decode runs a token sequence one token at a time with fewer slots
than experts (hits, misses and evictions through the library's planner); the GPU lookup must
report exactly the selected experts without a slot. Prefill runs with a permuted slot
assignment (each slot's fp16 staging exponent is derived from the expert it holds, so the
staged weights are those of the resident layer), and in expert tiles when the chunk selects more experts than there are slots
(Mference "Prefill": experts streamed in tiles through the slot cache). An absent slot must
be counted and must not be read outside the slab.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_moe_bit_amd import binding as B
from quantized_moe_bit_amd import synth
from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

pytestmark = pytest.mark.gpu

DIMS = synth.Dims(d_model=1024, n_experts=32, top_k=4, d_expert=256, d_shared=512)


def say(msg):
    print(f"[slots] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def check_oracle(y, lay, x, what, tol=2e-3):
    """y (device, [T, d]) against the oracle's layer output on x (bf16 bits [T, d])."""
    ref, _ = oracle.layer_forward(lay, x)
    got = y.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.max(np.abs(got - ref)) / rms
    assert np.all(np.isfinite(got)) and err <= tol, f"{what}: max|err| {err:.2e} rms"
    return err


def test_decode_sequence_through_slots():
    lay = synth.gen_layer(DIMS, 91, router="normal", zipf_s=1.0)
    x, _, _ = synth.gen_tokens(DIMS, 40, 91)
    ref = DeviceLayer(lay, max_tokens=16)
    sl = DeviceLayer(lay, max_tokens=16, n_slots=8)
    xd = tokens_to_device(x)
    fills = hits = 0
    y_all = torch.empty((x.shape[0], DIMS.d_model), dtype=torch.float32, device="cuda:0")
    for t in range(x.shape[0]):
        xt = xd[t:t + 1]
        r = sl.route(xt)
        idx = r["idx"]
        table = sl.slot_cache.table()
        sel = idx.cpu().numpy().ravel()
        want_missing = np.unique(sel[table[sel] < 0])
        np.testing.assert_array_equal(sl.missing(idx), want_missing, err_msg=f"token {t} lookup")
        n = sl.ensure(sel)
        fills += n
        hits += len(np.unique(sel)) - n
        y = sl.decode(xt, y_all[t:t + 1])
        y_ref = ref.decode(xt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(y), bits(y_ref), err_msg=f"token {t}")
    err = check_oracle(y_all, lay, x, "slot decode sequence")
    # two tokens per call: the union of their experts must be resident
    for t in range(0, 8, 2):
        sel = sl.route(xd[t:t + 2])["idx"].cpu().numpy().ravel()
        sl.ensure(sel)
        np.testing.assert_array_equal(bits(sl.decode(xd[t:t + 2])), bits(ref.decode(xd[t:t + 2])))
    assert B.moe_slot_faults(sl.handle) == 0
    assert fills > 8 and hits > 0
    say(f"decode: {x.shape[0]} tokens through 8 of 32 slots, {fills} fills, {hits} hits, bit-identical, "
        f"oracle max|err| {err:.2e} rms")
    sl.close()
    ref.close()


def test_prefill_with_permuted_slots():
    lay = synth.gen_layer(DIMS, 92, router="normal")
    x, _, _ = synth.gen_tokens(DIMS, 150, 92)
    ref = DeviceLayer(lay, max_tokens=150)
    sl = DeviceLayer(lay, max_tokens=150, n_slots=DIMS.n_experts)
    for e in reversed(range(DIMS.n_experts)):   # expert E-1 takes slot 0, ... expert 0 slot E-1
        sl.ensure([e])
    assert list(sl.slot_cache.table()) == list(reversed(range(DIMS.n_experts)))
    xd = tokens_to_device(x)
    y = sl.prefill(xd)
    y_ref = ref.prefill(xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    assert B.moe_slot_faults(sl.handle) == 0
    err = check_oracle(y, lay, x, "permuted-slot prefill")
    say(f"prefill: 150 tokens with a permuted slot table, bit-identical, oracle max|err| {err:.2e} rms")
    sl.close()
    ref.close()


def test_absent_slot_is_counted_and_contained():
    lay = synth.gen_layer(DIMS, 93, router="normal")
    x, _, _ = synth.gen_tokens(DIMS, 20, 93)
    ref = DeviceLayer(lay, max_tokens=20)
    sl = DeviceLayer(lay, max_tokens=20, n_slots=DIMS.n_experts)
    sl.ensure(list(range(DIMS.n_experts)))
    xd = tokens_to_device(x)
    sel = sl.route(xd[:1])["idx"].cpu().numpy().ravel()
    table = sl.slot_cache.table()
    broken = table.copy()
    broken[sel[0]] = -1
    sl.set_slot_table(broken)
    np.testing.assert_array_equal(sl.missing(sl.route(xd[:1])["idx"]), [sel[0]])
    sl.decode(xd[:1])
    sl.prefill(xd)
    torch.cuda.synchronize()
    assert B.moe_slot_faults(sl.handle, reset=True) > 0
    sl.set_slot_table(table)
    y = sl.decode(xd[:1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), bits(ref.decode(xd[:1])))
    assert B.moe_slot_faults(sl.handle) == 0
    say("absent slot: counted by decode and prefill, nothing read outside the slab; table restored")
    sl.close()
    ref.close()


@pytest.mark.parametrize("overlap", [False, True])
def test_prefill_in_expert_tiles(overlap):
    """More experts in the chunk than slots: tiles of at most n_slots experts filled in line, or
    (overlap) tiles of at most half the slots whose fills run on a copy stream while the previous
    tile's kernels run (Mference system design, "Prefill")."""
    lay = synth.gen_layer(DIMS, 94, router="normal", zipf_s=0.5)
    x, _, _ = synth.gen_tokens(DIMS, 150, 94)
    ref = DeviceLayer(lay, max_tokens=150)
    sl = DeviceLayer(lay, max_tokens=150, n_slots=8)
    xd = tokens_to_device(x)
    y_ref = ref.prefill(xd)
    y, tiles, fills = sl.prefill_tiled(xd, overlap=overlap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), bits(y_ref))
    err = check_oracle(y, lay, x, "tiled prefill")
    per = 4 if overlap else 8
    assert tiles >= 3 and fills >= per * (tiles - 1)
    y2, tiles2, fills2 = sl.prefill_tiled(xd, overlap=overlap)   # residents of the last tile are reused first
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y2), bits(y_ref))
    assert fills2 < fills
    assert B.moe_slot_faults(sl.handle) == 0
    # a decode between chunks, then another chunk: fills wait for everything queued before them
    sl.ensure(sl.route(xd[:1])["idx"].cpu().numpy().ravel())
    y_d = sl.decode(xd[:1])
    y3, _, _ = sl.prefill_tiled(xd, overlap=overlap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y3), bits(y_ref))
    np.testing.assert_array_equal(bits(y_d), bits(ref.decode(xd[:1])))
    assert B.moe_slot_faults(sl.handle) == 0
    say(f"prefill (overlap {overlap}): 150 tokens through 8 slots in {tiles} expert tiles ({fills} fills, "
        f"then {fills2}), bit-identical, oracle max|err| {err:.2e} rms")
    with pytest.raises(B.MoeError):
        B.moe_prefill_tile(ref.handle, 150, 0)   # a layer without slots
    # tiles and the combine belong to the chunk the layer routed last
    for call in (lambda: B.moe_prefill_tile(sl.handle, 149, 0), lambda: B.moe_prefill_combine(sl.handle, 149, y)):
        with pytest.raises(B.MoeError) as ei:
            call()
        assert ei.value.status == B.MOE_E_INVALID
    sl.ensure(sl.route(xd[:1])["idx"].cpu().numpy().ravel())
    sl.decode(xd[:1])   # the decode path reuses the workspace: no routed chunk afterwards
    for call in (lambda: B.moe_prefill_tile(sl.handle, 150, 0), lambda: B.moe_prefill_combine(sl.handle, 150, y)):
        with pytest.raises(B.MoeError) as ei:
            call()
        assert ei.value.status == B.MOE_E_INVALID
    sl.close()
    ref.close()
