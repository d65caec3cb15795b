"""Device-side layer object: repacks canonical weights (host, via moe_repack), places
them in device memory with PyTorch, creates the C-ABI handle and calls its entry
points. Marshalling only; every step of the layer runs in libmoe.so's kernels."""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device, non_blocking=False)


class DeviceLayer:
    """One MoE layer resident on a GPU. `layer` is a canonical-layout synth.Layer."""

    def __init__(self, layer, max_tokens: int, device="cuda:0", n_slots: Optional[int] = None, flags: int = 0):
        """n_slots: keep the routed experts in that many slots (expert slot cache): every
        expert's device-layout bytes stay in pinned host memory and `ensure` fills slots.
        flags: MOE_FLAG_* of moe_layer_create."""
        self.dims_py = layer.dims
        self.device = torch.device(device)
        D = layer.dims
        self._keep = {}
        self.n_slots = n_slots
        self._slot_src = {}
        q = {}
        specs = {
            "router": (layer.router, 8, 1, D.n_experts, D.d_model),
            "gate": (layer.gate, 4, D.n_experts, D.d_expert, D.d_model),
            "up": (layer.up, 4, D.n_experts, D.d_expert, D.d_model),
            "down": (layer.down, 4, D.n_experts, D.d_model, D.d_expert),
            "sh_gate": (layer.sh_gate, 4, 1, D.d_shared, D.d_model),
            "sh_up": (layer.sh_up, 4, 1, D.d_shared, D.d_model),
            "sh_down": (layer.sh_down, 4, 1, D.d_model, D.d_shared),
        }
        for name, (m, bits, n, o, i) in specs.items():
            if getattr(m, "fmt", "affine") == "q4_0":
                c, s = B.moe_repack_q4_0(n, o, i, m.codes)
            else:
                c, s = B.moe_repack(bits, n, o, i, m.codes, m.scales, m.biases)
            if n_slots is not None and name in ("gate", "up", "down"):
                # slab of n_slots experts; each expert's bytes stay on the host
                pc, ps = c.size // n, s.size // n
                hc = torch.from_numpy(c).pin_memory()
                hs = torch.from_numpy(s.view(np.int32)).pin_memory()
                tc = torch.zeros(n_slots * pc, dtype=torch.uint8, device=self.device)
                ts = torch.zeros(n_slots * ps, dtype=torch.int32, device=self.device)
                self._slot_src[name] = (hc, hs, pc, ps)
            else:
                tc, ts = _dev(c, self.device), _dev(s.view(np.int32), self.device)
            self._keep[name] = (tc, ts)
            q[name] = B.moe_qmat(tc.data_ptr(), ts.data_ptr())
        vecs = {"logit_bias": None if layer.logit_bias is None else layer.logit_bias.astype(np.float32),
                "router_scale": None if layer.router_scale is None else layer.router_scale.view(np.int16),
                "per_expert_scale": None if layer.per_expert_scale is None else layer.per_expert_scale.view(np.int16),
                "post_ffn_norm": None if layer.post_ffn_norm is None else layer.post_ffn_norm.view(np.int16),
                "layer_scalar": None if layer.layer_scalar is None else
                np.asarray(layer.layer_scalar, np.uint16).reshape(1).view(np.int16),
                "shared_gate": None if getattr(layer, "shared_gate", None) is None else layer.shared_gate.view(np.int16)}
        for name, v in vecs.items():
            if v is not None:
                self._keep[name] = _dev(v, self.device)
        if n_slots is not None:
            self.slot_cache = B.SlotCache(D.n_experts, n_slots)
            self._table_host = torch.full((D.n_experts,), -1, dtype=torch.int32).pin_memory()
            self._table = self._table_host.to(self.device)
        w = self._weights(q)
        self.dims = B.moe_dims(D.d_model, D.n_experts, D.top_k, D.d_expert, D.d_shared, D.group, D.router_bits,
                               D.expert_bits, max_tokens, B.FORMATS[getattr(D, "expert_format", "affine")])
        self.max_tokens = max_tokens
        self.weights = w   # the moe_weights the handle was created with
        self.handle = B.moe_layer_create(self.dims, w, flags)

    def replicate(self) -> "DeviceLayer":
        """A copy of this layer in fresh device memory (same values, new addresses, new handle)."""
        if self.n_slots is not None:
            raise NotImplementedError("replicate() of a layer with expert slots")
        other = DeviceLayer.__new__(DeviceLayer)
        other.dims_py = self.dims_py
        other.device = self.device
        other.n_slots = None
        other._slot_src = {}
        other.max_tokens = self.max_tokens
        other._keep = {}
        q = {}
        for name, v in self._keep.items():
            if name in self._VECS:
                other._keep[name] = v.clone()
            else:
                tc, ts = v[0].clone(), v[1].clone()
                other._keep[name] = (tc, ts)
                q[name] = B.moe_qmat(tc.data_ptr(), ts.data_ptr())
        w = other._weights(q)
        other.dims = B.moe_dims(*[getattr(self.dims, f) for f, _ in B.moe_dims._fields_])
        other.handle = B.moe_layer_create(other.dims, w, 0)
        return other

    _VECS = ("logit_bias", "router_scale", "per_expert_scale", "post_ffn_norm", "layer_scalar", "shared_gate")

    def _weights(self, q) -> "B.moe_weights":
        vec = {n: (self._keep[n].data_ptr() if n in self._keep else None) for n in self._VECS}
        if self.n_slots is not None:
            vec["expert_slot"] = self._table.data_ptr()
            vec["n_slots"] = self.n_slots
        return B.moe_weights(**q, **vec)

    # -------------------------------------------------------------- expert slots
    def ensure(self, experts, stream=None) -> int:
        """Make the listed experts resident: plan with the library's slot planner, copy the
        fills from pinned host memory into their slots and upload the slot table, all on the
        current stream (so later calls on it see them). Returns the number of fills."""
        _, fills = self.slot_cache.plan(experts)
        self._fill(fills)
        if fills:
            # a fresh pinned staging copy per update: an earlier upload may still be in flight
            tab = torch.from_numpy(self.slot_cache.table()).pin_memory()
            self._table.copy_(tab, non_blocking=True)
            self._staged = tab
        return len(fills)

    def _fill(self, fills):
        """Copy the planned fills [(expert, slot)] from pinned host memory into their slots (on
        the current stream)."""
        for e, sl in fills:
            for name, (hc, hs, pc, ps) in self._slot_src.items():
                tc, ts = self._keep[name]
                tc[sl * pc:(sl + 1) * pc].copy_(hc[e * pc:(e + 1) * pc], non_blocking=True)
                ts[sl * ps:(sl + 1) * ps].copy_(hs[e * ps:(e + 1) * ps], non_blocking=True)

    def _upload_table(self, table: np.ndarray, keep: list):
        tab = torch.from_numpy(np.ascontiguousarray(table, np.int32)).pin_memory()
        self._table.copy_(tab, non_blocking=True)
        keep.append(tab)

    def prefill_tiled(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, overlap: bool = False,
                      tile_experts: Optional[int] = None):
        """Prefill one chunk through the slot cache in expert tiles (Mference system design,
        "Prefill"): route once, then per tile make its experts resident and run its projections
        with a table that maps only them, then combine.

        overlap: tiles of at most half the slots (tile_experts overrides), and the fills of tile
        i + 1 run on a copy stream while tile i's kernels run: tile i + 1 is planned with tile i's
        experts protected (they keep their slots), every fill waits for the last queued kernel
        that read its slot, and a tile's kernels wait for its own fills. Without overlap, tiles of
        up to n_slots experts and fills in line on the compute stream.
        Returns (y, tiles, fills)."""
        T = x.shape[0]
        D = self.dims_py
        comp = torch.cuda.current_stream(self.device)
        if y is None:
            y = torch.empty((T, D.d_model), dtype=torch.float32, device=self.device)
        counts = torch.empty(D.n_experts, dtype=torch.int32, device=self.device)
        B.moe_prefill_route(self.handle, x, T, counts)
        used = np.nonzero(counts.cpu().numpy())[0]
        table = self.slot_cache.table()
        order = [int(e) for e in used if table[e] >= 0] + [int(e) for e in used if table[e] < 0]
        cap = tile_experts or (max(1, self.n_slots // 2) if overlap else self.n_slots)
        tiles = [order[i:i + cap] for i in range(0, len(order), cap)] or [[]]
        fills, staged, prev = 0, [], []
        if overlap:
            if getattr(self, "_copy_stream", None) is None:
                self._copy_stream = torch.cuda.Stream(self.device)
            copy = self._copy_stream
            # fills may only start after everything queued before this chunk (earlier calls read
            # the slots too)
            start = torch.cuda.Event()
            start.record(comp)
            copy.wait_event(start)
            reader = {}   # slot -> event after the last queued tile kernels that read it
        for ti, tile in enumerate(tiles):
            slot_of, plan_fills = self.slot_cache.plan(tile, protect=prev if overlap else ())
            if plan_fills:
                if overlap:
                    with torch.cuda.stream(copy):
                        for _, sl in plan_fills:
                            if sl in reader:
                                copy.wait_event(reader[sl])
                        self._fill(plan_fills)
                        done = torch.cuda.Event()
                        done.record(copy)
                    comp.wait_event(done)
                else:
                    self._fill(plan_fills)
            fills += len(plan_fills)
            active = np.full(D.n_experts, -1, np.int32)
            active[tile] = slot_of
            self._upload_table(active, staged)
            B.moe_prefill_tile(self.handle, T, ti)
            if overlap:
                ev = torch.cuda.Event()
                ev.record(comp)
                for sl in slot_of:
                    reader[sl] = ev
            prev = tile
        self._upload_table(self.slot_cache.table(), staged)
        self._staged_tiles = staged
        B.moe_prefill_combine(self.handle, T, y)
        return y, len(tiles), fills

    def set_slot_table(self, table: np.ndarray):
        """Upload an expert-to-slot table as is (synchronously; tests of absent slots)."""
        self._table.copy_(torch.from_numpy(np.ascontiguousarray(table, np.int32)))

    def missing(self, idx: torch.Tensor) -> np.ndarray:
        """Distinct selected experts without a slot, from the GPU slot lookup (synchronizes)."""
        out = torch.empty(1 + self.dims_py.n_experts, dtype=torch.int32, device=self.device)
        B.moe_slot_lookup(self.handle, idx, idx.shape[0], out)
        o = out.cpu().numpy()
        return o[1:1 + o[0]]

    def tail(self):
        """Device tensors of the layer tail (post-FFN norm weight, layer scalar); None where absent."""
        return self._keep.get("post_ffn_norm"), self._keep.get("layer_scalar")

    def weight_bytes(self) -> int:
        tot = 0
        for v in self._keep.values():
            for t in (v if isinstance(v, tuple) else (v,)):
                tot += t.numel() * t.element_size()
        return tot

    def close(self):
        if getattr(self, "handle", None):
            B.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------- calls
    def route(self, x: torch.Tensor, with_logits=True, with_grouping=True):
        T = x.shape[0]
        D = self.dims_py
        dev = self.device
        idx = torch.empty((T, D.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, D.top_k), dtype=torch.float32, device=dev)
        lg = torch.empty((T, D.n_experts), dtype=torch.float32, device=dev) if with_logits else None
        off = torch.empty(D.n_experts + 1, dtype=torch.int32, device=dev) if with_grouping else None
        perm = torch.empty(T * D.top_k, dtype=torch.int32, device=dev) if with_grouping else None
        B.moe_route(self.handle, x, T, idx, w, lg, off, perm)
        return dict(idx=idx, w=w, logits=lg, offsets=off, perm=perm)

    def decode(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.dims_py.d_model), dtype=torch.float32, device=self.device)
        B.moe_forward_decode(self.handle, x, T, y)
        return y

    def prefill(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.dims_py.d_model), dtype=torch.float32, device=self.device)
        B.moe_forward_prefill(self.handle, x, T, y)
        return y


def tokens_to_device(x_bits: np.ndarray, device="cuda:0") -> torch.Tensor:
    """bf16 bit patterns (uint16 [T, d]) -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(device)
