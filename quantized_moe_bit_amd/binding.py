"""Thin Python binding of the C ABI in include/moe.h (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls and does no
computation of its own: all of the layer runs in the gfx950 kernels of
libmoe.so. PyTorch supplies device memory and the HIP stream. If the library
is missing, loading fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

from . import build as _build

LIB_PATH = _build.LIB
_lib = None

(MOE_OK, MOE_E_INVALID, MOE_E_SHAPE, MOE_E_QUANT, MOE_E_ALIGN, MOE_E_CAPACITY, MOE_E_NOMEM, MOE_E_DEVICE,
 MOE_E_NONFINITE) = range(9)
MOE_MAX_DECODE_TOKENS = 16
MOE_FLAG_CHECK_FINITE = 0x1


def MOE_FLAG_WS_BUDGET_MIB(n: int) -> int:
    return (int(n) & 0xFFFFFF) << 8


KERNEL_NAMES = []


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: {status_str(status)}: {msg}")
        self.status = status


class moe_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("d_model", "n_experts", "top_k", "d_expert", "d_shared", "group",
                                         "router_bits", "expert_bits", "max_tokens", "expert_format")]


MOE_FORMAT_AFFINE_G64 = 0
MOE_FORMAT_Q4_0 = 1
FORMATS = {"affine": MOE_FORMAT_AFFINE_G64, "q4_0": MOE_FORMAT_Q4_0}


class moe_qmat(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("sb", C.c_void_p)]


class moe_weights(C.Structure):
    _fields_ = [(n, moe_qmat) for n in ("router", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")] + \
               [(n, C.c_void_p) for n in ("logit_bias", "router_scale", "per_expert_scale", "post_ffn_norm",
                                           "layer_scalar", "shared_gate", "expert_slot")] + \
               [("n_slots", C.c_int32)]


class moe_host_qmat(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p)]


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_moe_bit_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.moe_build_id.restype = C.c_char_p
        L.moe_build_id.argtypes = []
        built, want = L.moe_build_id().decode(), _build.source_hash()
        if built != want:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (build id {built[:16]}, sources "
                               f"{want[:16]}): rebuild it with `python -m quantized_moe_bit_amd.build`")
        vp, i32, st = C.c_void_p, C.c_int32, C.c_int
        sig = {
            "moe_layer_create": (st, [C.POINTER(moe_dims), C.POINTER(moe_weights), C.c_uint32, C.POINTER(vp)]),
            "moe_layer_destroy": (None, [vp]),
            "moe_route": (st, [vp, vp, i32, vp, vp, vp, vp, vp, vp]),
            "moe_forward_decode": (st, [vp, vp, i32, vp, vp]),
            "moe_forward_prefill": (st, [vp, vp, i32, vp, vp]),
            "moe_last_routing": (st, [vp, i32, vp, vp, vp]),
            "moe_forward_decode_noalloc": (st, [C.POINTER(moe_dims), C.POINTER(moe_weights), vp, i32, vp, vp]),
            "moe_stack_glue": (st, [vp, vp, vp, vp, vp, vp, i32, i32, vp]),
            "moe_stack_forward_decode": (st, [C.POINTER(vp), i32, vp, i32, vp, vp, vp, vp]),
            "moe_stack_plan_create": (st, [C.POINTER(vp), i32, vp, i32, vp, vp, vp, C.POINTER(vp)]),
            "moe_stack_plan_run": (st, [vp, vp]),
            "moe_stack_plan_destroy": (None, [vp]),
            "moe_packed_bytes": (C.c_size_t, [i32, i32, i32, i32, i32]),
            "moe_repack": (st, [i32, i32, i32, i32, C.POINTER(moe_host_qmat), vp, vp]),
            "moe_unrepack": (st, [i32, i32, i32, i32, vp, vp, vp, vp, vp]),
            "moe_repack_q4_0": (st, [i32, i32, i32, vp, vp, vp]),
            "moe_unrepack_q4_0": (st, [i32, i32, i32, vp, vp, vp]),
            "moe_status_str": (C.c_char_p, [st]),
            "moe_last_error": (C.c_char_p, []),
            "moe_profile_enable": (st, [vp, i32]),
            "moe_profile_read": (st, [vp, i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
            "moe_profile_reset": (st, [vp]),
            "moe_kernel_name": (C.c_char_p, [i32]),
            "moe_slot_lookup": (st, [vp, vp, i32, vp, vp]),
            "moe_prefill_route": (st, [vp, vp, i32, vp, vp]),
            "moe_prefill_tile": (st, [vp, i32, i32, vp]),
            "moe_prefill_combine": (st, [vp, i32, vp, vp]),
            "moe_slot_faults": (st, [vp, i32, C.POINTER(C.c_int32), vp]),
            "moe_slot_cache_create": (st, [i32, i32, C.POINTER(vp)]),
            "moe_slot_cache_destroy": (None, [vp]),
            "moe_slot_cache_plan": (st, [vp, vp, i32, vp, vp, vp, C.POINTER(C.c_int32)]),
            "moe_slot_cache_plan_protected": (st, [vp, vp, i32, vp, i32, vp, vp, vp, C.POINTER(C.c_int32)]),
            "moe_slot_cache_table": (st, [vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
        KERNEL_NAMES.clear()
        i = 0
        while True:
            nm = L.moe_kernel_name(i)
            if nm is None:
                break
            KERNEL_NAMES.append(nm.decode())
            i += 1
    return _lib


def status_str(s: int) -> str:
    return lib().moe_status_str(s).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what, moe_last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------------------- entry points
def moe_layer_create(dims: moe_dims, weights: moe_weights, flags: int = 0) -> int:
    h = C.c_void_p()
    _check(lib().moe_layer_create(C.byref(dims), C.byref(weights), flags, C.byref(h)), "moe_layer_create")
    return h.value


def moe_layer_destroy(handle: int) -> None:
    lib().moe_layer_destroy(handle)


def moe_route(handle, x, T, topk_idx, topk_w, logits=None, expert_offsets=None, pair_perm=None, stream=None):
    _check(lib().moe_route(handle, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(expert_offsets),
                           _ptr(pair_perm), _stream(stream)), "moe_route")


def moe_forward_decode(handle, x, T, y, stream=None):
    _check(lib().moe_forward_decode(handle, _ptr(x), T, _ptr(y), _stream(stream)), "moe_forward_decode")


def moe_forward_prefill(handle, x, T, y, stream=None):
    _check(lib().moe_forward_prefill(handle, _ptr(x), T, _ptr(y), _stream(stream)), "moe_forward_prefill")


def moe_forward_decode_noalloc(dims: moe_dims, weights: moe_weights, x, T, y, stream=None):
    _check(lib().moe_forward_decode_noalloc(C.byref(dims), C.byref(weights), _ptr(x), T, _ptr(y), _stream(stream)),
           "moe_forward_decode_noalloc")


def moe_last_routing(handle, T, idx, w, stream=None):
    _check(lib().moe_last_routing(handle, T, _ptr(idx), _ptr(w), _stream(stream)), "moe_last_routing")


def moe_build_id() -> str:
    return lib().moe_build_id().decode()


def moe_stack_glue(h, y, h_next, x_next, T, d, stream=None, post=None, scalar=None):
    _check(lib().moe_stack_glue(_ptr(h), _ptr(y), _ptr(post), _ptr(scalar), _ptr(h_next), _ptr(x_next), T, d,
                                _stream(stream)), "moe_stack_glue")


def moe_stack_forward_decode(handles, h, T, x_buf, y_buf, h_buf, stream=None):
    arr = (C.c_void_p * len(handles))(*handles)
    _check(lib().moe_stack_forward_decode(arr, len(handles), _ptr(h), T, _ptr(x_buf), _ptr(y_buf), _ptr(h_buf),
                                          _stream(stream)), "moe_stack_forward_decode")


def moe_stack_plan_create(handles, h, T, x_buf, y_buf, h_buf) -> int:
    """The stack call recorded once as a graph; returns the plan handle."""
    arr = (C.c_void_p * len(handles))(*handles)
    out = C.c_void_p()
    _check(lib().moe_stack_plan_create(arr, len(handles), _ptr(h), T, _ptr(x_buf), _ptr(y_buf), _ptr(h_buf),
                                       C.byref(out)), "moe_stack_plan_create")
    return out.value


def moe_stack_plan_run(plan, stream=None):
    _check(lib().moe_stack_plan_run(plan, _stream(stream)), "moe_stack_plan_run")


def moe_stack_plan_destroy(plan):
    lib().moe_stack_plan_destroy(plan)


def moe_packed_bytes(bits, n_mats, out_dim, in_dim, part) -> int:
    return int(lib().moe_packed_bytes(bits, n_mats, out_dim, in_dim, part))


def moe_repack(bits, n_mats, out_dim, in_dim, codes, scales, biases):
    """Canonical host arrays -> (device-layout codes uint8, sb uint32), both host NumPy arrays."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    biases = np.ascontiguousarray(biases, np.uint16)
    nc = moe_packed_bytes(bits, n_mats, out_dim, in_dim, 0)
    ns = moe_packed_bytes(bits, n_mats, out_dim, in_dim, 1)
    out_c = np.empty(max(nc, 1), np.uint8)
    out_s = np.empty(max(ns // 4, 1), np.uint32)
    src = moe_host_qmat(codes.ctypes.data, scales.ctypes.data, biases.ctypes.data)
    _check(lib().moe_repack(bits, n_mats, out_dim, in_dim, C.byref(src), out_c.ctypes.data, out_s.ctypes.data),
           "moe_repack")
    return out_c, out_s


def moe_unrepack(bits, n_mats, out_dim, in_dim, codes_dev, sb_dev):
    G = in_dim // 64
    codes = np.empty((n_mats, out_dim, in_dim * bits // 8), np.uint8)
    scales = np.empty((n_mats, out_dim, G), np.uint16)
    biases = np.empty((n_mats, out_dim, G), np.uint16)
    codes_dev = np.ascontiguousarray(codes_dev, np.uint8)
    sb_dev = np.ascontiguousarray(sb_dev, np.uint32)
    _check(lib().moe_unrepack(bits, n_mats, out_dim, in_dim, codes_dev.ctypes.data, sb_dev.ctypes.data,
                              codes.ctypes.data, scales.ctypes.data, biases.ctypes.data), "moe_unrepack")
    return codes, scales, biases


def moe_repack_q4_0(n_mats, out_dim, in_dim, blocks):
    """Q4_0 host blocks (uint8, 18 bytes per 32 inputs) -> (device-layout codes uint8, sb uint32)."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    nc = moe_packed_bytes(4, n_mats, out_dim, in_dim, 0)
    ns = moe_packed_bytes(4, n_mats, out_dim, in_dim, 1)
    out_c = np.empty(max(nc, 1), np.uint8)
    out_s = np.empty(max(ns // 4, 1), np.uint32)
    _check(lib().moe_repack_q4_0(n_mats, out_dim, in_dim, blocks.ctypes.data, out_c.ctypes.data, out_s.ctypes.data),
           "moe_repack_q4_0")
    return out_c, out_s


def moe_unrepack_q4_0(n_mats, out_dim, in_dim, codes_dev, sb_dev):
    blocks = np.empty((n_mats, out_dim, in_dim // 32 * 18), np.uint8)
    codes_dev = np.ascontiguousarray(codes_dev, np.uint8)
    sb_dev = np.ascontiguousarray(sb_dev, np.uint32)
    _check(lib().moe_unrepack_q4_0(n_mats, out_dim, in_dim, codes_dev.ctypes.data, sb_dev.ctypes.data,
                                   blocks.ctypes.data), "moe_unrepack_q4_0")
    return blocks


def moe_profile_enable(handle, on: bool):
    _check(lib().moe_profile_enable(handle, int(bool(on))), "moe_profile_enable")


def moe_profile_read(handle, kernel_id: int):
    ms, n = C.c_double(), C.c_int64()
    _check(lib().moe_profile_read(handle, kernel_id, C.byref(ms), C.byref(n)), "moe_profile_read")
    return ms.value, n.value


def moe_profile_reset(handle):
    _check(lib().moe_profile_reset(handle), "moe_profile_reset")


def kernel_id(name: str) -> int:
    lib()
    return KERNEL_NAMES.index(name)


def moe_slot_lookup(handle, idx, T, missing, stream=None):
    _check(lib().moe_slot_lookup(handle, _ptr(idx), T, _ptr(missing), _stream(stream)), "moe_slot_lookup")


def moe_slot_faults(handle, reset=False, stream=None) -> int:
    n = C.c_int32()
    _check(lib().moe_slot_faults(handle, int(bool(reset)), C.byref(n), _stream(stream)), "moe_slot_faults")
    return n.value


class SlotCache:
    """The library's host-side slot planner (least-frequently used, recency as the tie-breaker)."""

    def __init__(self, n_experts: int, n_slots: int):
        h = C.c_void_p()
        _check(lib().moe_slot_cache_create(n_experts, n_slots, C.byref(h)), "moe_slot_cache_create")
        self.handle, self.n_experts, self.n_slots = h.value, n_experts, n_slots

    def plan(self, experts, protect=()):
        """-> (slot of each listed expert, [(expert, slot) fills]); protected experts keep their slots"""
        e = np.ascontiguousarray(np.asarray(experts, np.int32).ravel())
        p = np.ascontiguousarray(np.asarray(list(protect), np.int32).ravel())
        n = e.shape[0]
        slot_of = np.empty(max(n, 1), np.int32)
        fe = np.empty(max(n, 1), np.int32)
        fs = np.empty(max(n, 1), np.int32)
        nf = C.c_int32()
        _check(lib().moe_slot_cache_plan_protected(self.handle, e.ctypes.data, n, p.ctypes.data if p.size else None,
                                                   p.shape[0], slot_of.ctypes.data, fe.ctypes.data, fs.ctypes.data,
                                                   C.byref(nf)), "moe_slot_cache_plan")
        return slot_of[:n].tolist(), list(zip(fe[:nf.value].tolist(), fs[:nf.value].tolist()))

    def table(self) -> np.ndarray:
        t = np.empty(self.n_experts, np.int32)
        _check(lib().moe_slot_cache_table(self.handle, t.ctypes.data), "moe_slot_cache_table")
        return t

    def close(self):
        if getattr(self, "handle", None):
            lib().moe_slot_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_prefill_route(handle, x, T, expert_counts=None, stream=None):
    _check(lib().moe_prefill_route(handle, _ptr(x), T, _ptr(expert_counts), _stream(stream)), "moe_prefill_route")


def moe_prefill_tile(handle, T, tile, stream=None):
    _check(lib().moe_prefill_tile(handle, T, tile, _stream(stream)), "moe_prefill_tile")


def moe_prefill_combine(handle, T, y, stream=None):
    _check(lib().moe_prefill_combine(handle, T, _ptr(y), _stream(stream)), "moe_prefill_combine")
