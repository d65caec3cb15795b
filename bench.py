#!/usr/bin/env python3
"""Benchmark of the quantized MoE FFN layer on one MI355X.

One step = one pass of the whole layer (router, top-8 + softmax, expert
gate/up + GeGLU, down, shared expert, weighted combine) over one batch of
synthetic input already resident in HBM. The headline workload is single-token
decode through one 2816-wide layer (128 experts, top-8, expert width 704,
shared width 2112). To measure HBM rather than the 256 MB Infinity Cache, each
step uses the next of --layers copies of the layer at distinct device addresses
and the next of 256 distinct tokens.

Prints one JSON line. Per-kernel durations for the roofline come from HIP events
the library records around each kernel launch on the same stream, during a
second pass over the same steps (so the headline timing carries no per-kernel
events). Also reports a 4096-token prefill chunk (MFMA utilisation) and the CPU
oracle timed on this host's cores on a bounded sample.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 / fp16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (vector, and matrix), TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "hbm_counters_decode_prefill.md")


def counter_traffic(kernel):
    """HBM bytes (read + written) per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when there is none or the kernel sources changed since it was taken."""
    import hashlib
    import re
    if not os.path.exists(COUNTER_SUMMARY):
        return None
    txt = open(COUNTER_SUMMARY).read()
    m = re.search(r"sha256 over ([^)]+)\):", txt)
    m_h = re.search(r"source_sha256: ([0-9a-f]{64})", txt)
    m_t = re.search(rf"traffic_bytes {kernel}: read (\d+) written (\d+)", txt)
    if not (m and m_h and m_t):
        return None
    h = hashlib.sha256()
    for src in (s.strip() for s in m.group(1).split(",")):
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != m_h.group(1):
        return None
    return int(m_t.group(1)) + int(m_t.group(2))


def qmat_bytes(out_dim, in_dim, bits):
    return out_dim * in_dim * bits // 8 + out_dim * (in_dim // 64) * 4


def decode_layer_bytes(D):
    """Weights one decode token streams once: router, k routed and the shared gate/up, down."""
    d, I, Is, E, k = D.d_model, D.d_expert, D.d_shared, D.n_experts, D.top_k
    return {"dec_router": qmat_bytes(E, d, 8),
            "dec_gateup": k * 2 * qmat_bytes(I, d, 4) + 2 * qmat_bytes(Is, d, 4),
            "dec_down": k * qmat_bytes(d, I, 4) + qmat_bytes(d, Is, 4)}


def decode_rotated(args, dev, name, K, W):
    """Decode of one token per call through --layers copies of a workload's layer (rotated, so the
    weights come from HBM), timed with events, then a second pass with per-kernel events."""
    import torch
    from quantized_moe_bit_amd import binding as B
    from quantized_moe_bit_amd import synth
    from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device
    wd = synth.WORKLOADS[name]
    D = wd.dims
    lay = synth.workload_layer(wd)
    base = DeviceLayer(lay, max_tokens=1, device=dev)
    copies = [base] + [base.replicate() for _ in range(args.layers - 1)]
    xt, _, _ = synth.gen_tokens(D, 256, wd.seed + 1000)
    xs = tokens_to_device(xt, dev)
    y = torch.empty((1, D.d_model), dtype=torch.float32, device=dev)

    def step(i):
        B.moe_forward_decode(copies[i % len(copies)].handle, xs[i % 256: i % 256 + 1], 1, y)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        step(W + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    for L in copies:
        B.moe_profile_reset(L.handle)
        B.moe_profile_enable(L.handle, True)
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    stage = decode_layer_bytes(D)
    kus = {}
    for kname in stage:
        tot, n = 0.0, 0
        for L in copies:
            m, c = B.moe_profile_read(L.handle, B.kernel_id(kname))
            tot += m
            n += c
        kus[kname] = 1000.0 * tot / max(n, 1)
    for L in copies:
        L.close()
    torch.cuda.empty_cache()
    btok = sum(stage.values())
    return {"tokens_per_s": round(1000.0 / ms, 1), "us_per_token": round(1000.0 * ms, 3),
            "bytes_per_token": btok, "hbm_gbs": round(btok / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(btok / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_us": {n: round(v, 3) for n, v in kus.items()},
            "kernels_gbs": {n: round(stage[n] / (kus[n] * 1e-6) / 1e9, 1) for n in stage}}


def q4_0_section(args, dev, K, W):
    """The 2816-wide layer with Q4_0 experts: 1-token decode (rotated copies) and a 4096-token
    prefill chunk. A Q4_0 block (18 bytes per 32 weights) streams the same 36 bytes per 64 weights
    as an affine group, so the decode byte counts are the affine ones."""
    log("Q4_0 experts: decode and 4096-token prefill")
    out = {"workload": "the 2816-wide layer (128 experts, top-8, widths 704 / 2112) with Q4_0 expert "
                       "matrices (fp16 d per 32 weights), 8-bit g64 router",
           "decode": decode_rotated(args, dev, "q4_0_decode", K, W)}
    if not args.no_prefill:
        out["prefill"] = prefill_section(args, dev, "q4_0_prefill4096",
                                         "prefill: 4096 tokens, Q4_0 experts, Zipf(1.3) logit skew, 2% tied tokens")[3]
    return out


def qwen_section(args, dev, K, W):
    """Decode (1 token, layer copies rotated) and 4096-token prefill of the 2048-wide,
    256-expert layer with a gated shared expert."""
    import torch
    from quantized_moe_bit_amd import binding as B
    from quantized_moe_bit_amd import synth
    from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device
    out = {}
    log("generating the 2048-wide 256-expert layer with a gated shared expert")
    D = synth.WORKLOADS["qwen_decode"].dims
    out["workload"] = ("layer d_model 2048, 256 experts, top-8, expert width 512, shared width 512 with a "
                       "sigmoid(g . x) gate, 8-bit g64 router, 4-bit g64 experts")
    out["decode"] = decode_rotated(args, dev, "qwen_decode", K, W)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_prefill:
        torch.cuda.empty_cache()
        wp = synth.WORKLOADS["qwen_prefill4096"]
        lp = synth.workload_layer(wp)
        xp, _, _ = synth.workload_tokens(wp, lp)
        T = wp.tokens
        P = DeviceLayer(lp, max_tokens=T, device=dev)
        xpd = tokens_to_device(xp, dev)
        yp = torch.empty((T, D.d_model), dtype=torch.float32, device=dev)
        for _ in range(2):
            B.moe_forward_prefill(P.handle, xpd, T, yp)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.prefill_steps):
            B.moe_forward_prefill(P.handle, xpd, T, yp)
        e1.record()
        torch.cuda.synchronize()
        msp = e0.elapsed_time(e1) / args.prefill_steps
        B.moe_profile_reset(P.handle)
        B.moe_profile_enable(P.handle, True)
        for _ in range(args.prefill_steps):
            B.moe_forward_prefill(P.handle, xpd, T, yp)
        torch.cuda.synchronize()
        pk = {}
        for kid, name in enumerate(B.KERNEL_NAMES):
            m, c = B.moe_profile_read(P.handle, kid)
            if c:
                pk[name] = round(1000.0 * m / c, 2)
        P.close()
        d, I, Is, k = D.d_model, D.d_expert, D.d_shared, D.top_k
        flops = 2.0 * (T * k * 2 * I * d + T * 2 * Is * d) + 2.0 * (T * k * d * I + T * d * Is)
        out["prefill"] = {"tokens": T, "routing": "Zipf(1.3) logit skew, 2% tied tokens",
                          "ms_per_step": round(msp, 4), "tokens_per_s": round(T / (msp * 1e-3), 1),
                          "mfma_tflops": round(flops / (msp * 1e-3) / 1e12, 2),
                          "mfma_frac": round(flops / (msp * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                          "kernels_us": pk}
    return out


def slot_section(dev, ntok=256):
    """Expert slot cache on the 2816-wide layer with Zipf(1.3) routing, one token per call:
    (a) every expert resident through a permuted slot table against the plain resident layer
    (the cost of the indirection); (b) 16 slots streamed from pinned host memory: per token
    route, GPU lookup of the missing experts (read back), plan, fills, forward."""
    import torch
    from quantized_moe_bit_amd import binding as B
    from quantized_moe_bit_amd import synth
    from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device
    wl = synth.WORKLOADS["prefill4096"]
    D = wl.dims
    log("generating the Zipf-routed 2816-wide layer for the slot cache")
    lay = synth.workload_layer(wl)
    x, _, _ = synth.workload_tokens(wl, lay, T=ntok)
    xd = tokens_to_device(x, dev)
    y = torch.empty((1, D.d_model), dtype=torch.float32, device=dev)
    out = {"workload": f"{ntok} Zipf(1.3)-routed tokens, one per call, through one 2816-wide layer "
                       "(128 experts, top-8)"}
    res = DeviceLayer(lay, max_tokens=1, device=dev)
    perm = DeviceLayer(lay, max_tokens=1, device=dev, n_slots=D.n_experts)
    for e in reversed(range(D.n_experts)):
        perm.ensure([e])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = {}
    for name, L in (("resident", res), ("all_in_slots", perm)):
        for i in range(20):
            B.moe_forward_decode(L.handle, xd[i:i + 1], 1, y)
        torch.cuda.synchronize()
        e0.record()
        for i in range(ntok):
            B.moe_forward_decode(L.handle, xd[i:i + 1], 1, y)
        e1.record()
        torch.cuda.synchronize()
        us[name] = 1000.0 * e0.elapsed_time(e1) / ntok
    out["decode_us_resident"] = round(us["resident"], 3)
    out["decode_us_all_in_slots"] = round(us["all_in_slots"], 3)
    res.close()
    perm.close()
    ss = DeviceLayer(lay, max_tokens=1, device=dev, n_slots=16)
    expert_bytes = 3 * qmat_bytes(D.d_expert, D.d_model, 4)
    fills = hits = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(ntok):
        r = ss.route(xd[i:i + 1], with_logits=False, with_grouping=False)
        miss = ss.missing(r["idx"])                   # GPU lookup, read back
        sel = r["idx"].cpu().numpy().ravel()
        n = ss.ensure(sel)
        assert n == len(miss)
        fills += n
        hits += len(np.unique(sel)) - n
        B.moe_forward_decode(ss.handle, xd[i:i + 1], 1, y)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert B.moe_slot_faults(ss.handle) == 0
    ss.close()
    # a 4096-token chunk through 16 slots in expert tiles: fills in line (tiles of 16 experts) and
    # overlapped with the previous tile's kernels (tiles of 8, fills on a copy stream); against the
    # same chunk with every expert resident (compute only) and the fills alone (copies only)
    wp = synth.WORKLOADS["prefill4096"]
    xp, _, _ = synth.workload_tokens(wp, lay)
    xpd = tokens_to_device(xp, dev)
    Tp = wp.tokens
    yp = torch.empty((Tp, D.d_model), dtype=torch.float32, device=dev)
    resident = DeviceLayer(lay, max_tokens=Tp, device=dev)
    for _ in range(2):
        resident.prefill(xpd, yp)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(3):
        resident.prefill(xpd, yp)
    torch.cuda.synchronize()
    compute_ms = 1000.0 * (time.perf_counter() - t1) / 3
    resident.close()
    tiled = {}
    for overlap in (False, True):
        pt = DeviceLayer(lay, max_tokens=Tp, device=dev, n_slots=16)
        pt.prefill_tiled(xpd, yp, overlap=overlap)
        torch.cuda.synchronize()
        walls, tl, fl = [], 0, 0
        for _ in range(3):
            t1 = time.perf_counter()
            _, tl, f = pt.prefill_tiled(xpd, yp, overlap=overlap)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t1)
            fl += f
        assert B.moe_slot_faults(pt.handle) == 0
        # the same number of expert fills alone: copies only, no kernels
        used = np.arange(D.n_experts)
        nf = max(1, round(fl / 3))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        pt._fill([(int(used[i % D.n_experts]), i % 16) for i in range(nf)])
        torch.cuda.synchronize()
        fill_ms = 1000.0 * (time.perf_counter() - t1)
        pt.close()
        tiled["overlapped" if overlap else "in_line"] = {
            "ms_per_chunk_host_inclusive": round(1000.0 * sorted(walls)[1], 3), "tiles": tl,
            "fills_per_chunk": round(fl / 3, 1), "fill_bytes_per_chunk": round(fl / 3 * expert_bytes),
            "fills_alone_ms": round(fill_ms, 3), "compute_alone_ms": round(compute_ms, 3),
            "sum_fills_and_compute_ms": round(fill_ms + compute_ms, 3)}
    out["prefill_4096_16_slots"] = dict(tiled, note="median of three chunks through the same cache after one; "
                                                    "fills from pinned host memory")
    out["streaming_16_slots"] = {
        "tokens_per_s_host_inclusive": round(ntok / wall, 1), "hit_rate": round(hits / max(hits + fills, 1), 4),
        "fills_per_token": round(fills / ntok, 3), "expert_bytes": expert_bytes,
        "fill_gbs_host_to_device": round(fills * expert_bytes / wall / 1e9, 2),
        "note": "wall clock per token includes the host readback of the missing list, planning and "
                "pinned-host-to-HBM fills"}
    return out


def prefill_section(args, dev, name, label):
    """One prefill chunk of a workload through one layer: chunk time over --prefill-steps calls after
    two warm-up calls, MFMA rate of the whole step and of each GEMM, and per-kernel durations from a
    second pass with the library's dispatch-attached events. Returns (layer, x on device, T, dict)."""
    import torch
    from quantized_moe_bit_amd import binding as B
    from quantized_moe_bit_amd import synth
    from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device
    wp = synth.WORKLOADS[name]
    D = wp.dims
    lp = synth.workload_layer(wp)
    xp, _, _ = synth.workload_tokens(wp, lp)
    T = wp.tokens
    P = DeviceLayer(lp, max_tokens=T, device=dev)
    xpd = tokens_to_device(xp, dev)
    yp = torch.empty((T, D.d_model), dtype=torch.float32, device=dev)
    for _ in range(2):
        B.moe_forward_prefill(P.handle, xpd, T, yp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.prefill_steps):
        B.moe_forward_prefill(P.handle, xpd, T, yp)
    e1.record()
    torch.cuda.synchronize()
    ms_pre = e0.elapsed_time(e1) / args.prefill_steps
    B.moe_profile_reset(P.handle)
    B.moe_profile_enable(P.handle, True)
    e0.record()
    for _ in range(args.prefill_steps):
        B.moe_forward_prefill(P.handle, xpd, T, yp)
    e1.record()
    torch.cuda.synchronize()
    ms_kpass = e0.elapsed_time(e1) / args.prefill_steps
    pk = {}
    for kid, kname in enumerate(B.KERNEL_NAMES):
        ms, c = B.moe_profile_read(P.handle, kid)
        if c:
            pk[kname] = 1000.0 * ms / c
    B.moe_profile_enable(P.handle, False)
    # weights the chunk streams: every expert it routes to, the shared expert and the router, once
    # each (a small chunk is bound by streaming them, not by the matrix cores)
    r = P.route(xpd, with_logits=False)
    torch.cuda.synchronize()
    n_used = int((np.diff(r["offsets"].cpu().numpy()) > 0).sum())
    P.close()
    d, I, Is, k = D.d_model, D.d_expert, D.d_shared, D.top_k
    wbytes = (n_used * (2 * qmat_bytes(I, d, 4) + qmat_bytes(d, I, 4)) + 2 * qmat_bytes(Is, d, 4)
              + qmat_bytes(d, Is, 4) + qmat_bytes(D.n_experts, d, 8))
    fl_gateup = 2.0 * (T * k * 2 * I * d + T * 2 * Is * d)
    fl_down = 2.0 * (T * k * d * I + T * d * Is)
    flops = fl_gateup + fl_down
    pre = {"workload": label,
           "tokens_per_s": round(T / (ms_pre * 1e-3), 1), "ms_per_step": round(ms_pre, 4),
           "mfma_flops_per_step": flops,
           "mfma_tflops": round(flops / (ms_pre * 1e-3) / 1e12, 2),
           "mfma_frac": round(flops / (ms_pre * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
           "kernels_us": {n: round(v, 2) for n, v in pk.items()},
           "kernels_sum_us": round(sum(pk.values()), 2),
           "kernels_pass_us_per_step": round(1000.0 * ms_kpass, 2),
           "experts_used": n_used, "weight_bytes_per_step": wbytes,
           "weight_gbs": round(wbytes / (ms_pre * 1e-3) / 1e9, 1),
           "weight_hbm_frac": round(wbytes / (ms_pre * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "note": "sustained back-to-back chunks lower the clock (the same chunk's GEMMs take up to ~25% "
                   "longer after a few chunks), so per-kernel times are compared with the step time of "
                   "their own instrumented pass"}
    for kname, fl in (("pre_gateup", fl_gateup), ("pre_down", fl_down)):
        if kname in pk:
            tf = fl / (pk[kname] * 1e-6) / 1e12
            pre["roofline_" + kname[4:]] = dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_PEAK_TFLOPS,
                                                 unit="TFLOP/s", frac=round(tf / MFMA_PEAK_TFLOPS, 4),
                                                 flops=fl, avg_us=round(pk[kname], 2))
    if "router" in pk:
        # fp32 fixed-order chains: on fp32 MFMA (matrix-core router) or as VALU fma chains (the
        # group-split router the library takes for small chunks); both peaks are 157.3 TFLOP/s
        E = D.n_experts
        valu = d // 64 <= 64 and -(-T // 64) * -(-E // 4) <= 512
        fl = 2.0 * T * E * d
        tf = fl / (pk["router"] * 1e-6) / 1e12
        pre["roofline_router"] = dict(bound="alu" if valu else "mfma", achieved=round(tf, 1), peak=FP32_PEAK_TFLOPS,
                                      unit="TFLOP/s", frac=round(tf / FP32_PEAK_TFLOPS, 4), flops=fl,
                                      avg_us=round(pk["router"], 2))
    return lp, xpd, T, pre


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=16, help="distinct-address layer copies the decode steps rotate over")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload (prefill-only runs)")
    ap.add_argument("--no-stack", action="store_true", help="skip the 30-layer decode stack workload")
    ap.add_argument("--stack-layers", type=int, default=0, help="layers of the stack workload (0: its 30)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prologue", action="store_true", help="skip the router prologue measurement")
    ap.add_argument("--no-qwen", action="store_true", help="skip the gated-shared-expert (Qwen 3.6 style) layer")
    ap.add_argument("--no-slots", action="store_true", help="skip the expert slot cache measurement")
    ap.add_argument("--no-q4-0", dest="no_q4_0", action="store_true", help="skip the Q4_0-expert layer")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this layer has no cross-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_moe_bit_amd import binding as B
    from quantized_moe_bit_amd import synth
    from quantized_moe_bit_amd.device import DeviceLayer, tokens_to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup

    # ------------------------------------------------------------------ decode workload
    if args.no_decode:
        args.layers, K = 1, 1
    wl = synth.WORKLOADS["decode"]
    D = wl.dims
    log("generating the 2816-wide layer")
    lay = synth.workload_layer(wl)
    base = DeviceLayer(lay, max_tokens=16, device=dev)   # 1-token steps; 16-token calls for the batch line
    layers = [base] + [base.replicate() for _ in range(args.layers - 1)]
    xt, _, _ = synth.gen_tokens(D, 256, wl.seed + 1000)
    xs = tokens_to_device(xt, dev)
    y = torch.empty((1, D.d_model), dtype=torch.float32, device=dev)
    ntok = xs.shape[0]

    def step(i):
        B.moe_forward_decode(layers[i % len(layers)].handle, xs[i % ntok: i % ntok + 1], 1, y)

    log(f"decode warmup {W}, timed {K} steps over {len(layers)} layer copies")
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        step(W + i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / K

    # the same layer copies with 16-token decode calls (batched decode, distinct tokens per call)
    xs16 = tokens_to_device(synth.gen_tokens(D, 16 * 16, wl.seed + 2000)[0], dev)
    y16 = torch.empty((16, D.d_model), dtype=torch.float32, device=dev)

    def step16(i):
        j = i % 16
        B.moe_forward_decode(layers[i % len(layers)].handle, xs16[16 * j:16 * j + 16], 16, y16)

    for i in range(W):
        step16(i)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(K):
        step16(W + i)
    ev1.record()
    torch.cuda.synchronize()
    ms_step16 = ev0.elapsed_time(ev1) / K

    # per-kernel durations: a second pass of the same steps with events attached to each kernel
    # dispatch on the layer's stream (they time the interval a kernel trace reports); the pass's own
    # step time is measured too, so the kernel sum is compared with a step of the same pass
    for L in layers:
        B.moe_profile_reset(L.handle)
        B.moe_profile_enable(L.handle, True)
    ev0.record()
    for i in range(K):
        step(W + i)
    ev1.record()
    torch.cuda.synchronize()
    ms_kpass = ev0.elapsed_time(ev1) / K
    kern = {}
    for kid, name in enumerate(B.KERNEL_NAMES):
        tot, n = 0.0, 0
        for L in layers:
            ms, c = B.moe_profile_read(L.handle, kid)
            tot += ms
            n += c
        if n:
            kern[name] = dict(avg_us=1000.0 * tot / n, launches=n)
    for L in layers:
        B.moe_profile_enable(L.handle, False)

    # algorithmic bytes per token (weights streamed, once each)
    d, I, Is, E, k = D.d_model, D.d_expert, D.d_shared, D.n_experts, D.top_k
    b_router = qmat_bytes(E, d, 8)
    b_gateup = k * 2 * qmat_bytes(I, d, 4) + 2 * qmat_bytes(Is, d, 4)
    b_down = k * qmat_bytes(d, I, 4) + qmat_bytes(d, Is, 4)
    b_token = b_router + b_gateup + b_down
    # algorithmic bytes of each decode launch: weights it streams once
    stage_bytes = {
        "dec_router": b_router,
        "dec_gateup": k * 2 * qmat_bytes(I, d, 4) + 2 * qmat_bytes(Is, d, 4),
        "dec_down": k * qmat_bytes(d, I, 4) + qmat_bytes(d, Is, 4),
    }
    assert sum(stage_bytes.values()) == b_token
    roofline = None
    timed = {n: v for n, v in kern.items() if n in stage_bytes}
    if timed:
        dom = max(timed, key=lambda n: timed[n]["avg_us"])
        achieved = stage_bytes[dom] / (timed[dom]["avg_us"] * 1e-6) / 1e9
        roofline = dict(kernel=dom, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                        unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=counter_traffic(dom),
                        algorithmic_bytes=stage_bytes[dom], avg_us=round(timed[dom]["avg_us"], 3))
    layer_gbs = b_token / (ms_step * 1e-3) / 1e9

    result = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA % of MI355X peak",
        "value": round(1000.0 / ms_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "decode: 1 token through one layer, d_model 2816, 128 experts, top-8, "
                               "expert width 704, shared width 2112, 8-bit g64 router, 4-bit g64 experts",
                   "tokens_per_step": 1, "layer_copies_rotated": len(layers), "distinct_tokens": ntok,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "decode_batch16": {"workload": "16 tokens per decode call through the same layer copies",
                           "tokens_per_s": round(16 * 1000.0 / ms_step16, 1), "us_per_call": round(1000.0 * ms_step16, 3)},
        "decode": {"bytes_per_token": b_token, "layer_hbm_gbs": round(layer_gbs, 1),
                   "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4), "host_wall_s": round(wall, 4),
                   "kernels_us": {n: round(v["avg_us"], 3) for n, v in kern.items()},
                   "kernels_sum_us": round(sum(v["avg_us"] for n, v in kern.items() if n in stage_bytes), 3),
                   "kernels_pass_us_per_step": round(1000.0 * ms_kpass, 3),
                   "kernels_gbs": {n: round(stage_bytes[n] / (v["avg_us"] * 1e-6) / 1e9, 1)
                                   for n, v in kern.items() if n in stage_bytes}},
    }

    def release_decode_copies():
        for L in layers:
            L.close()
        layers.clear()
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ prefill chunks (4096 and 512 tokens)
    if not args.no_prefill:
        release_decode_copies()
        log("generating the 4096-token Zipf prefill workload")
        lp, xpd, T, pre = prefill_section(args, dev, "prefill4096",
                                          "prefill: 4096 tokens, one 2816-wide layer, Zipf(1.3) logit skew, 2% tied tokens")
        result["prefill"] = pre
        ms_pre = pre["ms_per_step"]
        yp = torch.empty((T, d), dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        log("generating the 512-token Zipf prefill workload")
        result["prefill512"] = prefill_section(args, dev, "prefill512",
                                               "prefill: 512 tokens, one 2816-wide layer, Zipf(1.1) logit skew")[3]
        if not args.no_prologue:
            # widened row: the same layer and tokens with the router prologue and per-expert scale
            rng = np.random.default_rng(7)
            lp.router_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, d).astype(np.float32))
            lp.per_expert_scale = synth.f32_to_bf16_bits(rng.uniform(0.5, 2.0, lp.dims.n_experts).astype(np.float32))
            PP = DeviceLayer(lp, max_tokens=T, device=dev)
            for _ in range(2):
                B.moe_forward_prefill(PP.handle, xpd, T, yp)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.prefill_steps):
                B.moe_forward_prefill(PP.handle, xpd, T, yp)
            e1.record()
            torch.cuda.synchronize()
            ms_pro = e0.elapsed_time(e1) / args.prefill_steps
            kid = B.kernel_id("router_prologue")
            B.moe_profile_reset(PP.handle)
            B.moe_profile_enable(PP.handle, True)
            for _ in range(args.prefill_steps):
                B.moe_forward_prefill(PP.handle, xpd, T, yp)
            torch.cuda.synchronize()
            ms_kp, n_kp = B.moe_profile_read(PP.handle, kid)
            B.moe_profile_reset(PP.handle)
            for _ in range(20):
                B.moe_forward_decode(PP.handle, xpd[:1], 1, yp[:1])
            torch.cuda.synchronize()
            ms_kd, n_kd = B.moe_profile_read(PP.handle, B.kernel_id("dec_router"))   # prologue fused in
            B.moe_profile_enable(PP.handle, False)
            us_p = 1000.0 * ms_kp / max(n_kp, 1)
            pro_bytes = 3 * 2 * T * d   # x read, u and the fp16 copy of x written (router_scale stays cached)
            result.setdefault("next_rows", {})["router_prologue"] = {
                "workload": "4096-token prefill chunk and 1-token decode through the 2816-wide layer with the "
                            "router prologue (rmsnorm without scale, router_scale / sqrt(d)) and per-expert scale",
                "prefill_ms_per_step": round(ms_pro, 4), "prefill_ms_without": round(ms_pre, 4),
                "prologue_us_prefill": round(us_p, 2), "prologue_bytes_prefill": pro_bytes,
                "prologue_gbs_prefill": round(pro_bytes / (us_p * 1e-6) / 1e9, 1),
                "decode_router_with_prologue_us": round(1000.0 * ms_kd / max(n_kd, 1), 2)}
            PP.close()

    # ------------------------------------------------------------------ widened row: gated shared expert
    if not args.no_qwen:
        release_decode_copies()
        result.setdefault("next_rows", {})["qwen_gated_shared"] = qwen_section(args, dev, K, W)

    # ------------------------------------------------------------------ widened row: Q4_0 experts
    if not args.no_q4_0:
        release_decode_copies()
        result.setdefault("next_rows", {})["q4_0_experts"] = q4_0_section(args, dev, K, W)

    # ------------------------------------------------------------------ widened row: expert slot cache
    if not args.no_slots:
        release_decode_copies()
        result.setdefault("next_rows", {})["expert_slots"] = slot_section(dev)

    # ------------------------------------------------------------------ 30-layer decode stack
    if not args.no_stack:
        release_decode_copies()
        ws = synth.WORKLOADS["stack"]
        NL = args.stack_layers or ws.layers
        log(f"generating the {NL}-layer decode stack")
        stack = []
        for l in range(NL):
            stack.append(DeviceLayer(synth.workload_layer(ws, l), max_tokens=1, device=dev))
        h0 = synth.gen_stack_tokens(ws.dims, ws.tokens, ws.seed)
        hd = tokens_to_device(h0, dev)
        xb = torch.empty((1, d), dtype=torch.int16, device=dev)
        yb = torch.empty((1, d), dtype=torch.float32, device=dev)
        hb = torch.empty_like(xb)
        handles = [L.handle for L in stack]
        for t in range(8):          # warmup on the first tokens, then the timed pass from h0
            B.moe_stack_forward_decode(handles, hd[t:t + 1], 1, xb, yb, hb)
        hd.copy_(tokens_to_device(h0, dev))
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for t in range(ws.tokens):
            B.moe_stack_forward_decode(handles, hd[t:t + 1], 1, xb, yb, hb)
        s1.record()
        torch.cuda.synchronize()
        ms_tok = s0.elapsed_time(s1) / ws.tokens
        st_bytes = NL * b_token
        result["stack"] = {"workload": f"decode stack: {NL} distinct 2816-wide layers, residual stream between "
                                       f"layers, {ws.tokens} consecutive tokens one at a time",
                           "tokens_per_s": round(1000.0 / ms_tok, 1), "ms_per_token": round(ms_tok, 4),
                           "us_per_layer": round(1000.0 * ms_tok / NL, 3), "bytes_per_token": st_bytes,
                           "hbm_gbs": round(st_bytes / (ms_tok * 1e-3) / 1e9, 1),
                           "hbm_frac": round(st_bytes / (ms_tok * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # the same stack recorded once (moe_stack_plan_create) and replayed per token on fixed
        # buffers, each token's stream copied into the plan's h first (the copy is timed too)
        hp = torch.empty_like(xb)
        plan = B.moe_stack_plan_create(handles, hp, 1, xb, yb, hb)
        for t in range(8):
            hp.copy_(hd[t:t + 1])
            B.moe_stack_plan_run(plan)
        torch.cuda.synchronize()
        s0.record()
        for t in range(ws.tokens):
            hp.copy_(hd[t:t + 1])
            B.moe_stack_plan_run(plan)
        s1.record()
        torch.cuda.synchronize()
        B.moe_stack_plan_destroy(plan)
        ms_plan = s0.elapsed_time(s1) / ws.tokens
        result["stack"]["recorded_plan"] = {
            "tokens_per_s": round(1000.0 / ms_plan, 1), "us_per_layer": round(1000.0 * ms_plan / NL, 3),
            "hbm_gbs": round(st_bytes / (ms_plan * 1e-3) / 1e9, 1),
            "note": "moe_stack_plan_run per token, including a device copy of the token's stream into the plan's h"}
        for L in stack:
            L.close()
        del stack
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ counter calibration copy
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n * 4

    # ------------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on a bounded sample")
        xs_host = xt
        done, t_start = 0, time.perf_counter()
        while True:
            chunk = xs_host[(done % ntok): (done % ntok) + 16]
            oracle.layer_forward(lay, chunk)
            done += chunk.shape[0]
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or el > 30:
                break
        result["cpu_baseline"] = {"value": round(done / el, 3), "unit": "tokens/s", "cores": oracle.get_threads(),
                                  "kind": "oracle",
                                  "sample": f"{done} decode tokens of the same 2816-wide layer (router, top-8, "
                                            f"8 experts + shared, combine) in {el:.1f} s"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
