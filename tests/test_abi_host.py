"""C-ABI boundary checks that need no GPU: the library loads and exports every
entry point include/moe.h declares, the lossless repack round-trips and follows
its documented layout, and argument validation rejects bad calls before any
device work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from quantized_moe_bit_amd import binding as B
from quantized_moe_bit_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_entry_point():
    lib = B.lib()
    names = declared_functions()
    assert {"moe_layer_create", "moe_route", "moe_forward_decode", "moe_forward_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert B.status_str(B.MOE_OK) == "MOE_OK"
    assert B.status_str(B.MOE_E_CAPACITY) == "MOE_E_CAPACITY"
    assert B.KERNEL_NAMES[:2] == ["router", "topk"]


@pytest.mark.parametrize("bits,n,o,i", [(4, 3, 64, 128), (4, 2, 96, 192), (8, 2, 5, 256), (4, 1, 32, 64)])
def test_repack_round_trip_is_bit_exact(bits, n, o, i):
    rng = np.random.default_rng(bits * 100 + o)
    codes = rng.integers(0, 256, size=(n, o, i * bits // 8), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=(n, o, i // 64), dtype=np.uint16)
    biases = rng.integers(0, 1 << 16, size=(n, o, i // 64), dtype=np.uint16)
    dc, ds = B.moe_repack(bits, n, o, i, codes, scales, biases)
    assert dc.nbytes == codes.nbytes and ds.nbytes == scales.nbytes * 2
    c2, s2, b2 = B.moe_unrepack(bits, n, o, i, dc, ds)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(b2, biases)


def test_repack_layout_matches_documentation():
    """Each code lands where the header says: tile (row block, group), lane, step, nibble."""
    n, o, i = 2, 64, 128
    G = i // 64
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(n, o, i // 2), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=(n, o, G), dtype=np.uint16)
    biases = rng.integers(0, 1 << 16, size=(n, o, G), dtype=np.uint16)
    dc, ds = B.moe_repack(4, n, o, i, codes, scales, biases)
    words = dc.view(np.uint32)
    for m in range(n):
        for row in range(o):
            for k in range(i):
                q = (codes[m, row, k // 2] >> (4 * (k % 2))) & 0xF
                rb, g, kk = row // 32, k // 64, k % 64
                s, rem = kk // 16, kk % 16
                half, j = rem // 8, rem % 8
                lane = (row % 32) + 32 * half
                nib = j // 2 if j % 2 == 0 else 4 + j // 2
                byte_off = m * o * i // 2 + (rb * G + g) * 1024 + lane * 16 + 4 * s
                assert (words[byte_off // 4] >> (4 * nib)) & 0xF == q
            for g in range(G):
                w = ds[m * o * G + ((row // 32) * G + g) * 32 + row % 32]
                assert w & 0xFFFF == scales[m, row, g] and w >> 16 == biases[m, row, g]


@pytest.mark.parametrize("n,o,i", [(3, 64, 128), (2, 96, 192), (1, 32, 64)])
def test_q4_0_repack_round_trip_is_bit_exact(n, o, i):
    """Any block bytes (scales included: NaN and infinite patterns are copied as bits)."""
    rng = np.random.default_rng(n * 1000 + o)
    blocks = rng.integers(0, 256, size=(n, o, i // 32 * 18), dtype=np.uint8)
    dc, ds = B.moe_repack_q4_0(n, o, i, blocks)
    assert dc.nbytes == B.moe_packed_bytes(4, n, o, i, 0) and ds.nbytes == B.moe_packed_bytes(4, n, o, i, 1)
    np.testing.assert_array_equal(B.moe_unrepack_q4_0(n, o, i, dc, ds), blocks)


def test_q4_0_repack_matches_the_affine_tile_layout():
    """Q4_0 codes land in the same tiles as the affine codes of the same elements (the affine
    layout is pinned element by element above), and each group's word holds its two blocks' d."""
    n, o, i = 2, 64, 192
    rng = np.random.default_rng(9)
    blocks = rng.integers(0, 256, size=(n, o, i // 32, 18), dtype=np.uint8)
    body = blocks[..., 2:]
    q = np.concatenate([body & 0x0F, body >> 4], axis=-1).reshape(n, o, i)   # element order
    canon = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)             # affine canonical packing
    G = i // 64
    zero = np.zeros((n, o, G), np.uint16)
    ac, _ = B.moe_repack(4, n, o, i, canon, zero, zero)
    dc, ds = B.moe_repack_q4_0(n, o, i, blocks.reshape(n, o, -1))
    np.testing.assert_array_equal(dc, ac)
    d = blocks[..., 0].astype(np.uint32) | (blocks[..., 1].astype(np.uint32) << 8)   # [n, o, i/32]
    for m in range(n):
        for row in range(o):
            for g in range(G):
                w = ds[m * o * G + ((row // 32) * G + g) * 32 + row % 32]
                assert w & 0xFFFF == d[m, row, 2 * g] and w >> 16 == d[m, row, 2 * g + 1]


def test_q4_0_repack_rejects_bad_arguments():
    z = np.zeros(8192, np.uint8)
    L = B.lib()
    for o, i, st in [(30, 64, B.MOE_E_SHAPE), (32, 96, B.MOE_E_SHAPE), (32, 32, B.MOE_E_SHAPE), (0, 64, B.MOE_E_SHAPE)]:
        out = np.zeros(4096, np.uint8)
        assert L.moe_repack_q4_0(1, o, i, z.ctypes.data, out.ctypes.data, out.ctypes.data) == st
        assert np.all(out == 0)
    assert L.moe_repack_q4_0(1, 32, 64, None, z.ctypes.data, z.ctypes.data) == B.MOE_E_INVALID
    assert L.moe_unrepack_q4_0(1, 32, 64, z.ctypes.data, None, z.ctypes.data) == B.MOE_E_INVALID


def test_packed_bytes_matches_canonical_sizes():
    d, I = 2816, 704
    per_proj = B.moe_packed_bytes(4, 1, I, d, 0) + B.moe_packed_bytes(4, 1, I, d, 1)
    assert per_proj == 1_115_136
    assert B.moe_packed_bytes(8, 1, 128, d, 0) + B.moe_packed_bytes(8, 1, 128, d, 1) == 382_976
    assert B.moe_packed_bytes(4, 1, 30, 128, 0) == 0          # 4-bit rows must tile by 32
    assert B.moe_packed_bytes(4, 1, 32, 100, 0) == 0          # inputs must group by 64


def test_repack_rejects_bad_arguments():
    z8 = np.zeros(64, np.uint8)
    z16 = np.zeros(4, np.uint16)
    for bits, o, i, st in [(3, 32, 64, B.MOE_E_QUANT), (4, 30, 64, B.MOE_E_SHAPE), (4, 32, 96, B.MOE_E_SHAPE)]:
        src = B.moe_host_qmat(z8.ctypes.data, z16.ctypes.data, z16.ctypes.data)
        out = np.zeros(4096, np.uint8)
        r = B.lib().moe_repack(bits, 1, o, i, C.byref(src), out.ctypes.data, out.ctypes.data)
        assert r == st
        assert np.all(out == 0)
    r = B.lib().moe_repack(4, 1, 32, 64, None, None, None)
    assert r == B.MOE_E_INVALID


def _dims(**kw):
    base = dict(d_model=256, n_experts=8, top_k=2, d_expert=128, d_shared=256, group=64, router_bits=8,
                expert_bits=4, max_tokens=16)
    base.update(kw)
    return B.moe_dims(**base)


def _weights(align=16, null=None):
    buf = (C.c_uint8 * 4096)()
    base = (C.addressof(buf) + 255) // 256 * 256
    q = {}
    for n, name in enumerate(("router", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")):
        p = base + 0 if name != null else 0
        q[name] = B.moe_qmat(p if p == 0 else p + (0 if align == 16 else 4), base)
    w = B.moe_weights(**q, logit_bias=None)
    w._buf = buf
    return w


@pytest.mark.parametrize("kw,status", [
    (dict(group=32), B.MOE_E_QUANT),
    (dict(router_bits=4), B.MOE_E_QUANT),
    (dict(expert_bits=8), B.MOE_E_QUANT),
    (dict(expert_format=2), B.MOE_E_QUANT),
    (dict(expert_format=-1), B.MOE_E_QUANT),
    (dict(d_model=200), B.MOE_E_SHAPE),
    (dict(d_expert=100), B.MOE_E_SHAPE),
    (dict(d_shared=0), B.MOE_E_SHAPE),
    (dict(top_k=9), B.MOE_E_SHAPE),
    (dict(top_k=0), B.MOE_E_SHAPE),
    (dict(n_experts=0), B.MOE_E_SHAPE),
    (dict(max_tokens=0), B.MOE_E_SHAPE),
])
def test_create_rejects_bad_dims_before_device_work(kw, status):
    h = C.c_void_p(0)
    r = B.lib().moe_layer_create(C.byref(_dims(**kw)), C.byref(_weights()), 0, C.byref(h))
    assert r == status, B.moe_last_error()
    assert h.value is None
    assert B.moe_last_error()


def test_create_rejects_chunks_with_more_routed_tiles_than_the_list_builder_holds():
    """A chunk of max_tokens tokens may hold ceil(T k / 128) + min(E, T k) routed row tiles; the
    GEMM work-list builder holds 16384 of them, so a layer whose bound exceeds that is refused
    (MOE_E_SHAPE) before any device work, while one just inside passes validation."""
    h = C.c_void_p(0)
    L = B.lib()
    big = dict(d_model=64, d_expert=64, d_shared=64, max_tokens=1 << 20)
    assert L.moe_layer_create(C.byref(_dims(top_k=2, **big)), C.byref(_weights()), 0, C.byref(h)) == B.MOE_E_SHAPE
    assert "routed row tiles" in B.moe_last_error()
    # top-1: 8192 + 8 tiles, within the bound; refused only by the tiny workspace budget
    assert L.moe_layer_create(C.byref(_dims(top_k=1, **big)), C.byref(_weights()), B.MOE_FLAG_WS_BUDGET_MIB(1),
                              C.byref(h)) == B.MOE_E_NOMEM
    assert h.value is None


def test_create_rejects_null_misaligned_and_flags():
    h = C.c_void_p(0)
    L = B.lib()
    assert L.moe_layer_create(C.byref(_dims()), C.byref(_weights(null="down")), 0, C.byref(h)) == B.MOE_E_INVALID
    assert L.moe_layer_create(C.byref(_dims()), C.byref(_weights(align=4)), 0, C.byref(h)) == B.MOE_E_ALIGN
    for bad_flags in (0x2, 0x80, 0x4):   # bits other than MOE_FLAG_CHECK_FINITE and the budget field
        assert L.moe_layer_create(C.byref(_dims()), C.byref(_weights()), bad_flags, C.byref(h)) == B.MOE_E_INVALID
    assert L.moe_layer_create(C.byref(_dims()), None, 0, C.byref(h)) == B.MOE_E_INVALID
    assert L.moe_layer_create(None, C.byref(_weights()), 0, C.byref(h)) == B.MOE_E_INVALID
    assert h.value is None


@pytest.mark.parametrize("d_model", [192, 256])
def test_workspace_budget_flag_refuses_before_allocating(d_model):
    """A workspace above the flags' budget is MOE_E_NOMEM, decided on the host before any
    allocation (no GPU here); d_model = 192 (a multiple of 64, not of 128) passes validation."""
    h = C.c_void_p(0)
    L = B.lib()
    dims = _dims(d_model=d_model, max_tokens=4096)
    for flags in (B.MOE_FLAG_WS_BUDGET_MIB(1), B.MOE_FLAG_WS_BUDGET_MIB(1) | B.MOE_FLAG_CHECK_FINITE):
        assert L.moe_layer_create(C.byref(dims), C.byref(_weights()), flags, C.byref(h)) == B.MOE_E_NOMEM
        assert "budget" in B.moe_last_error()
    assert h.value is None


def test_binding_refuses_a_library_built_from_other_sources(monkeypatch):
    """The library carries a hash of the sources it was built from; a loader refuses a stale one."""
    from quantized_moe_bit_amd import build as hb
    assert B.moe_build_id() == hb.source_hash()
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(hb, "source_hash", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="other sources"):
        B.lib()


def test_noalloc_decode_refuses_scratch_beyond_its_static_array():
    """The handle-free decode's scratch lives in a 1 MiB static device array: the widest layer at
    16 tokens needs more and is refused on the host, before any device call (no GPU here)."""
    L = B.lib()
    fake = (C.c_uint8 * 64)()
    p = (C.addressof(fake) + 15) // 16 * 16
    dims = _dims(d_model=8192, n_experts=1024, top_k=16, d_expert=1536, d_shared=4096, max_tokens=16)
    w = _weights()
    assert L.moe_forward_decode_noalloc(C.byref(dims), C.byref(w), p, 16, p, None) == B.MOE_E_CAPACITY
    assert "scratch" in B.moe_last_error()
    assert L.moe_forward_decode_noalloc(C.byref(dims), C.byref(w), p, 17, p, None) == B.MOE_E_CAPACITY
    assert L.moe_forward_decode_noalloc(C.byref(_dims(d_model=200)), C.byref(w), p, 1, p, None) == B.MOE_E_SHAPE
    assert L.moe_forward_decode_noalloc(None, C.byref(w), p, 1, p, None) == B.MOE_E_INVALID
    assert L.moe_forward_decode_noalloc(C.byref(_dims()), C.byref(w), p, 0, p, None) == B.MOE_OK   # no-op


def test_calls_reject_null_layer_and_bad_sizes():
    L = B.lib()
    assert L.moe_forward_decode(None, None, 1, None, None) == B.MOE_E_INVALID
    assert L.moe_forward_prefill(None, None, 1, None, None) == B.MOE_E_INVALID
    assert L.moe_route(None, None, 1, None, None, None, None, None, None) == B.MOE_E_INVALID
    assert L.moe_stack_glue(None, None, None, None, None, None, -1, 16, None) == B.MOE_E_SHAPE
    assert L.moe_stack_glue(None, None, None, None, None, None, 0, 16, None) == B.MOE_OK      # T = 0 is a no-op
    assert L.moe_stack_glue(None, None, None, None, None, None, 2, 16, None) == B.MOE_E_INVALID
    assert L.moe_stack_glue(None, None, None, None, None, None, 2, 12, None) == B.MOE_E_SHAPE     # d % 8
    assert L.moe_stack_glue(None, None, None, None, None, None, 2, 8200, None) == B.MOE_E_SHAPE   # d > 8192
    assert L.moe_profile_enable(None, 1) == B.MOE_E_INVALID
    one_null = (C.c_void_p * 1)(None)
    assert L.moe_stack_forward_decode(None, 1, None, 1, None, None, None, None) == B.MOE_E_INVALID
    assert L.moe_stack_forward_decode(one_null, 0, None, 1, None, None, None, None) == B.MOE_E_INVALID
    assert L.moe_stack_forward_decode(one_null, 1, None, 1, None, None, None, None) == B.MOE_E_INVALID
    # the recorded stack: argument checks before any stream or capture exists
    plan = C.c_void_p(1)
    assert L.moe_stack_plan_create(None, 1, None, 1, None, None, None, C.byref(plan)) == B.MOE_E_INVALID
    assert plan.value is None   # *out is cleared on error
    assert L.moe_stack_plan_create(one_null, 0, None, 1, None, None, None, C.byref(plan)) == B.MOE_E_INVALID
    assert L.moe_stack_plan_create(one_null, 1, None, 0, None, None, None, C.byref(plan)) == B.MOE_E_SHAPE
    assert L.moe_stack_plan_create(one_null, 1, None, 1, None, None, None, C.byref(plan)) == B.MOE_E_INVALID
    assert L.moe_stack_plan_create(one_null, 1, None, 1, None, None, None, None) == B.MOE_E_INVALID
    assert L.moe_stack_plan_run(None, None) == B.MOE_E_INVALID
    L.moe_stack_plan_destroy(None)
    # expert slots and tiled prefill: argument checks happen before anything touches a device
    assert L.moe_slot_lookup(None, None, 1, None, None) == B.MOE_E_INVALID
    assert L.moe_slot_faults(None, 0, None, None) == B.MOE_E_INVALID
    assert L.moe_prefill_route(None, None, 1, None, None) == B.MOE_E_INVALID
    assert L.moe_prefill_tile(None, 1, 0, None) == B.MOE_E_INVALID
    assert L.moe_prefill_combine(None, 1, None, None) == B.MOE_E_INVALID
    assert L.moe_last_routing(None, 1, None, None, None) == B.MOE_E_INVALID
    assert B.status_str(B.MOE_E_NONFINITE) == "MOE_E_NONFINITE"
    out = C.c_void_p()
    assert L.moe_slot_cache_create(8, 0, C.byref(out)) == B.MOE_E_SHAPE
    assert L.moe_slot_cache_create(0, 1, C.byref(out)) == B.MOE_E_SHAPE
    assert L.moe_slot_cache_create(8, 2, None) == B.MOE_E_INVALID
    assert L.moe_slot_cache_table(None, None) == B.MOE_E_INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_header_and_library_serve_a_plain_c99_program(tmp_path):
    """tests/c/abi_from_c.c, built by gcc as strict C99 against include/moe.h and linked to the
    library, runs the host-side calls (sizes, repack round trip, argument errors, create's
    dimension checks) with no Python in between."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    B.lib()   # the library exists and matches its sources
    libdir = os.path.dirname(B.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", libdir, "-lmoe",
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI host checks passed" in r.stdout
