"""Benchmark of the MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gemma4_class]
                    [--backward [--recompute-h] | --mxfp8] [--no-cpu-baseline] [--no-configs]
                    [--no-vendor-yardstick] [--stage-json PATH]

One step = one pass of the whole forward hot path over one batch: route,
permute, grouped GEMM 1 (prefused wi, SwiGLU epilogue), grouped GEMM 2 (wo),
combine. The timed loop calls the library's stage entry points in exactly
the order and form moe_ffn_fwd uses, with HIP events between launches on the
stream the kernels run on, so every kernel's duration is measured inside the
timed region. Inputs are resident in HBM before timing starts. Prints ONE
JSON line.

Forward only is the inference path: the permute builds the expert-sorted
index and GEMM 1 reads the token rows of x in place through it. With
--backward (DeepSeek-V3-shaped workload) the forward materialises the sorted
rows and the fp32 gate/up values for the backward, and the step also runs
the layer backward as moe_ffn_bwd runs it (combine-bwd, dWo, NT GEMM +
SwiGLU-bwd, dWi, NT GEMM, permute-bwd), each launch timed, and, where the
router is learned, the router backward (logit gradients from dtopk_w, dWr,
and dx += dlogits . Wr^T onto the layer's dx).
With --mxfp8 the forward runs its grouped GEMMs on MXFP8 operands: each token
row of x is quantized once and GEMM 1 reads the codes through sorted_slot,
GEMM 1's SwiGLU epilogue writes its output as MXFP8 for GEMM 2, and the
expert weights are quantized beforehand (weight preparation, outside the
timed step).
With --recompute-h the forward keeps no fp32 gate/up values and the backward
recomputes them with one more GEMM1 (the saved bytes are reported).

The bf16 forward line also carries `vendor_dense_gemm`: the vendor library's
dense GEMM of the same size and FLOPs as each grouped GEMM, timed after the
step as context for the roofline fraction (skip with --no-vendor-yardstick).

Unless --no-configs is given, the line also carries `configs`: the other
workloads measured the same way after the headline one (tiny, mid_skewed, the
Zipf token sweep and the DeepSeek-V3-shaped forward+backward), each with its
step time, tokens/s and every stage's time against its roofline floor.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 matrix cores (the router's fma chains run on them)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_ffn_group_amd", "csrc", "gemm.hip")
METRIC = "MoE FFN layer tokens/s + achieved bf16 MFMA TFLOP/s, 128 experts top-8"
# the other workloads of the line's `configs`, with their step counts
CONFIGS = [("tiny", False, 100), ("mid_skewed", False, 50), ("sweep_zipf_T1024", False, 50),
           ("sweep_zipf_T2048", False, 50), ("sweep_zipf_T4096", False, 30), ("sweep_zipf_T8192", False, 30),
           ("deepseek_v3_shape", True, 5)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gemma4_class")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--mxfp8", action="store_true",
                    help="forward with MXFP8 grouped GEMMs (activations quantized in the step, weights beforehand)")
    ap.add_argument("--recompute-h", action="store_true",
                    help="with --backward: the forward keeps no h and the backward recomputes it (full remat)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="measure the headline workload only")
    ap.add_argument("--no-vendor-yardstick", action="store_true",
                    help="skip timing the vendor library's dense GEMMs of the same sizes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--stage-json", default=None, help="also write per-stage details to this file")
    return ap.parse_args()


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def tf(flop, ms):
    return flop / (ms * 1e-3) / 1e12


def gb(b, ms):
    return b / (ms * 1e-3) / 1e9


def stage_entry(ms, flop=0.0, nbytes=0.0, fpeak=PEAK_BF16_TFLOPS, declared=None):
    """A stage's time against its roofline floor max(flop / peak, bytes / HBM peak). `declared` fixes the
    bound the stage is priced against (the headline's stages keep the bound each kernel is designed for)."""
    t_f = flop / (fpeak * 1e12) * 1e3 if flop else 0.0
    t_b = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3 if nbytes else 0.0
    bound = declared or ("mfma" if t_f >= t_b else "hbm")
    d = dict(ms=ms, bound=bound)
    if bound == "mfma":
        d.update(achieved=tf(flop, ms), peak=fpeak, unit="TFLOP/s")
    else:
        d.update(achieved=gb(nbytes, ms), peak=PEAK_HBM_GBS, unit="GB/s")
    d["frac"] = d["achieved"] / d["peak"]
    if flop:
        d["flop"] = flop
    if nbytes:
        d["bytes"] = nbytes
    return d


def measure(wl, dev, steps, warmup, bwd=False, remat=False, mx=False, flush_combine=False, fused_check=True):
    """Run the workload's step `warmup` + `steps` times on `dev`; every launch bracketed by HIP events on
    the stream it runs on. Returns the step time, per-stage times and the stages' roofline entries."""
    import numpy as np
    import torch

    import mixture_experts_ffn_group_amd as moe
    import workloads
    from mixture_experts_ffn_group_amd import _lib

    T, emb, mlp, E, k, S = wl.T, wl.emb, wl.mlp, wl.E, wl.k, wl.S
    inp = workloads.make_inputs(wl, device=dev)
    x, wi, wo, wr, bias, logits = inp["x"], inp["wi"], inp["wo"], inp["wr"], inp["bias"], inp["logits_in"]
    moe.query_support(T, emb, mlp, E, k)
    stream = torch.cuda.current_stream(dev)
    L = _lib.lib()
    shp = _lib.shape(T, emb, mlp, E, k)
    P = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    st = C.c_void_p(stream.cuda_stream)

    # buffers (allocated once, outside the timed region)
    saved = sv = moe.alloc_saved(T, emb, mlp, E, k, dev, keep_h=not remat)
    y = torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.workspace_bytes(T, emb, mlp, E, k), dtype=torch.uint8, device=dev)
    pws = torch.empty(max(16, int(L.moe_permute_workspace_bytes(C.byref(shp)))), dtype=torch.uint8, device=dev)
    router_bwd = bwd and wr is not None
    if bwd:
        dy = inp["dy"]
        bws = torch.empty(moe.workspace_bytes(T, emb, mlp, E, k, backward=True, recompute_h=remat),
                          dtype=torch.uint8, device=dev)
        grads = dict(dx=torch.empty((T, emb), dtype=torch.bfloat16, device=dev),
                     dwi=torch.empty_like(wi), dwo=torch.empty_like(wo),
                     dtopk_w=torch.empty((T, k), dtype=torch.float32, device=dev))
        # the backward's activations, as moe_ffn_bwd carves them from its workspace
        d_o = torch.empty((S, emb), dtype=torch.bfloat16, device=dev)
        dh = torch.empty((S, 2 * mlp), dtype=torch.bfloat16, device=dev)
        dxs = torch.empty((S, emb), dtype=torch.bfloat16, device=dev)
        hr = torch.empty((S, 2 * mlp), dtype=torch.float32, device=dev) if remat else None
        a_tmp = torch.empty((S, mlp), dtype=torch.bfloat16, device=dev) if remat else None
    if router_bwd:
        rbws = torch.empty(max(16, int(L.moe_route_bwd_workspace_bytes(C.byref(shp)))), dtype=torch.uint8,
                           device=dev)
        grads["dwr"] = torch.empty((emb, E), dtype=torch.float32, device=dev)
        grads["dbias"] = torch.empty(E, dtype=torch.float32, device=dev) if bias is not None else None

    # Inference (forward only) runs the path moe_ffn_fwd takes without a saved set: the permute builds
    # the index only and GEMM1 gathers the x rows through sorted_slot. With the backward the forward
    # materialises xs and h, which the backward reads.
    gather = not bwd
    rows = _lib.MoeGemmRows(P(sv["sorted_slot"]), S, k, None) if gather else None
    if mx:
        # MXFP8 operands: weights quantized once (weight preparation, outside the timed step), activations in it
        wiq, wis = moe.mx_quantize_weight(wi)       # [E, 2mlp, emb], [E, emb/64, 2mlp, 4]
        woq, wos = moe.mx_quantize_weight(wo)       # [E, emb, mlp], [E, mlp/64, emb, 4]
        xq = torch.empty((T, emb), dtype=torch.uint8, device=dev)   # token rows, read by GEMM 1 through sorted_slot
        xqs = torch.empty((emb // 64, T, 4), dtype=torch.uint8, device=dev)
        aq = torch.empty((S, mlp), dtype=torch.uint8, device=dev)
        aqs = torch.empty((mlp // 64, S, 4), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    route = ("route", lambda: L.moe_route(C.byref(shp), None if logits is not None else P(x), P(wr), P(bias),
                                          P(logits), P(sv["topk_idx"]), P(sv["topk_w"]), st))
    combine = ("combine", lambda: L.moe_combine(C.byref(shp), P(sv["o"]), P(sv["slot_row"]), P(sv["topk_w"]),
                                                P(y), st))
    if mx:
        calls = [
            route,
            ("permute", lambda: L.moe_permute(C.byref(shp), P(x), P(sv["topk_idx"]), P(sv["group_sizes"]),
                                              P(sv["group_offsets"]), P(sv["sorted_slot"]), P(sv["slot_row"]),
                                              None, P(pws), pws.numel(), st)),
            # each token row quantized once; GEMM 1 reads its codes and scales in place through sorted_slot
            ("quantize_x", lambda: L.moe_mx_quantize_rows(P(x), T, emb, None, 1, T, P(xq), P(xqs), st)),
            # GEMM 1 writes its SwiGLU output as MXFP8 directly (the operand of GEMM 2); no bf16 copy
            ("gemm1_swiglu", lambda: L.moe_grouped_gemm_mx(1, P(xq), P(xqs), T, P(sv["sorted_slot"]), k, P(wiq),
                                                           P(wis), P(sv["group_offsets"]), E, S, emb, 2 * mlp,
                                                           None, P(aq), P(aqs), st)),
            ("gemm2", lambda: L.moe_grouped_gemm_mx(0, P(aq), P(aqs), S, None, 1, P(woq), P(wos),
                                                    P(sv["group_offsets"]), E, S, mlp, emb, P(sv["o"]), None,
                                                    None, st)),
            combine,
        ]
    else:
        calls = [
            route,
            ("permute", lambda: L.moe_permute(C.byref(shp), P(x), P(sv["topk_idx"]), P(sv["group_sizes"]),
                                              P(sv["group_offsets"]), P(sv["sorted_slot"]), P(sv["slot_row"]),
                                              None if gather else P(sv["xs"]), P(pws), pws.numel(), st)),
            ("gemm1_swiglu", lambda: L.moe_grouped_gemm(0, 1, P(x) if gather else P(sv["xs"]), P(wi), None,
                                                        P(sv["h"]) if bwd else None, P(sv["group_offsets"]), E, S,
                                                        emb, 2 * mlp, C.byref(rows) if gather else None,
                                                        P(sv["a"]), st)),
            ("gemm2", lambda: L.moe_grouped_gemm(0, 0, P(sv["a"]), P(wo), None, None, P(sv["group_offsets"]), E, S,
                                                 mlp, emb, None, P(sv["o"]), st)),
            combine,
        ]
    if bwd:
        go = sv["group_offsets"]
        dgrows = _lib.MoeGemmRows(P(sv["sorted_slot"]), S, k, P(sv["topk_w"]))
        hsrc = hr if remat else sv["h"]
        calls += [
            # do (the permutation part) and dtopk_w (the reduction part)
            ("combine_bwd", lambda: L.moe_combine_bwd(C.byref(shp), P(dy), P(sv["o"]), P(sv["slot_row"]),
                                                      P(sv["topk_w"]), P(d_o), P(grads["dtopk_w"]), st)),
            ("wgrad_dwo", lambda: L.moe_grouped_gemm_wgrad(P(sv["a"]), P(d_o), P(go), E, S, mlp, emb,
                                                           P(grads["dwo"]), st)),
        ]
        if remat:
            calls.append(("recompute_h", lambda: L.moe_grouped_gemm(0, 1, P(sv["xs"]), P(wi), None, P(hr), P(go), E,
                                                                    S, emb, 2 * mlp, None, P(a_tmp), st)))
        calls += [
            # da = w * (dy . wo[e]^T) with dy rows read in place, then the SwiGLU backward into dh
            ("gemm_dh", lambda: L.moe_grouped_gemm(1, 2, P(dy), P(wo), P(hsrc), None, P(go), E, S, emb, mlp,
                                                   C.byref(dgrows), P(dh), st)),
            ("wgrad_dwi", lambda: L.moe_grouped_gemm_wgrad(P(sv["xs"]), P(dh), P(go), E, S, emb, 2 * mlp,
                                                           P(grads["dwi"]), st)),
            ("gemm_dxs", lambda: L.moe_grouped_gemm(1, 0, P(dh), P(wi), None, None, P(go), E, S, 2 * mlp, emb, None,
                                                    P(dxs), st)),
            ("permute_bwd", lambda: L.moe_combine(C.byref(shp), P(dxs), P(sv["slot_row"]), None, P(grads["dx"]),
                                                  st)),
        ]
    if router_bwd:
        calls.append(("route_bwd", lambda: L.moe_route_bwd(C.byref(shp), P(x), P(wr), P(sv["topk_idx"]),
                                                           P(sv["topk_w"]), P(grads["dtopk_w"]),
                                                           P(sv["sorted_slot"]), P(sv["group_offsets"]),
                                                           P(grads["dwr"]), P(grads["dbias"]), P(grads["dx"]),
                                                           P(rbws), rbws.numel(), st)))

    def run_step(events=None):
        for i, (name, f) in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            rc = f()
            if rc != 0:
                raise _lib.MoeError(rc, name, L.moe_last_error_detail().decode())
        if events is not None:
            events[len(calls)].record(stream)

    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    # The step time: K steps of the launches alone, bracketed by synchronizations.
    t0 = time.perf_counter()
    for s in range(steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The stage breakdown: K more steps with an event on the stream between the launches (the event
    # writes sit between the kernels, so this pass is not the one the step time is taken from).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        run_step(evs[s])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)]))
                for i, (name, _) in enumerate(calls)}

    # the fused entry points over the same buffers, as a cross-check of the staged timing
    fused_ms = bwd_fused_ms = None
    if fused_check:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if mx:
            wq = dict(wi_codes=wiq, wi_scales=wis, wo_codes=woq, wo_scales=wos, mlp=mlp)
            mws = torch.empty(int(L.moe_workspace_bytes_mx(C.byref(shp))), dtype=torch.uint8, device=dev)
            f = lambda: moe.ffn_fwd_mx(x, wq, k, wr=wr, bias=bias, logits=logits, workspace=mws, out=y)  # noqa: E731
        elif not bwd:
            f = lambda: moe.ffn_fwd(x, wi, wo, k, wr=wr, bias=bias, logits=logits, workspace=ws, out=y)  # noqa: E731
        else:
            def f():
                rc = L.moe_ffn_bwd(C.byref(shp), P(dy), C.byref(moe._saved_struct(sv)), P(wi), P(wo), P(grads["dx"]),
                                   P(grads["dwi"]), P(grads["dwo"]), P(grads["dtopk_w"]), P(bws), bws.numel(), st)
                if rc != 0:
                    raise _lib.MoeError(rc, "moe_ffn_bwd", L.moe_last_error_detail().decode())
        for _ in range(2):
            f()
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        if bwd and not mx:
            bwd_fused_ms = e0.elapsed_time(e1) / steps
        else:
            fused_ms = e0.elapsed_time(e1) / steps

    # The bf16 forward entry captured once in a HIP graph and replayed: the same kernels without the host's
    # per-launch cost, which is what limits the small workloads (the entry allocates nothing and records no
    # memset, so it can be captured as it is).
    graph_ms = None
    if fused_check and not bwd and not mx:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            f()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream(dev)
        e0.record(cur)
        for _ in range(steps):
            graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        del graph

    # The combine again, alone, with the 256 MB MALL (Infinity Cache) flushed before each launch: in the step
    # it reads o right after GEMM 2 wrote it, so part of o may still be in the MALL there. The flush writes a
    # 512 MB buffer and then reads it back, so that its own dirty lines are written back before the launch.
    comb_cold_ms = None
    if flush_combine:
        comb_call = dict(calls)["combine"]
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for c0, c1 in cold_evs:
            flush.fill_(1)
            flush.view(torch.int32).sum()
            c0.record(stream)
            rc = comb_call()
            c1.record(stream)
            if rc != 0:
                raise _lib.MoeError(rc, "combine", L.moe_last_error_detail().decode())
        torch.cuda.synchronize()
        comb_cold_ms = float(np.mean([c0.elapsed_time(c1) for c0, c1 in cold_evs]))
        del flush

    gs = saved["group_sizes"].cpu().numpy()
    e_nz = int((gs > 0).sum())
    ms_step = wall * 1e3 / steps

    # algorithmic work per launch (each non-empty expert's weights read once, activations once)
    g1_flop, g2_flop = 4.0 * S * emb * mlp, 2.0 * S * mlp * emb
    a_rows_bytes = T * emb * 2 if gather else S * emb * 2  # GEMM1's A: x read in place, or the sorted copy
    g1_bytes = a_rows_bytes + e_nz * emb * 2 * mlp * 2 + S * mlp * 2 + (S * 2 * mlp * 4 if bwd else 0)
    g2_bytes = S * mlp * 2 + e_nz * mlp * emb * 2 + S * emb * 2
    perm_bytes = 12 * S if gather else T * emb * 2 + S * emb * 2 + 12 * S
    comb_bytes = S * emb * 2 + 8 * S + T * emb * 2
    gpeak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    if mx:  # fp8 operands plus one scale byte per 32 elements (a dword per 64 in the padded layout)
        g1_bytes = T * emb * 17 // 16 + e_nz * emb * 2 * mlp * 17 // 16 + S * mlp * 17 // 16
        g2_bytes = S * mlp * 17 // 16 + e_nz * mlp * emb * 17 // 16 + S * emb * 2
        qx_bytes = T * emb * 2 + T * emb * 17 // 16      # x read once, token codes and scales written
    route_flop = 0.0 if logits is not None else 2.0 * T * emb * E
    route_bytes = (T * E * 4 if logits is not None else T * emb * 2 + emb * E * 4) + 8 * S

    stages = {
        "route": stage_entry(stage_ms["route"], route_flop, route_bytes, PEAK_FP32_MFMA_TFLOPS,
                             declared="mfma" if route_flop else "hbm"),
        "permute": dict(stage_entry(stage_ms["permute"], 0.0, perm_bytes, declared="hbm"),
                        rows="index only; GEMM1 gathers the x rows" if gather else "rows copied to xs"),
        "gemm1_swiglu": stage_entry(stage_ms["gemm1_swiglu"], g1_flop, g1_bytes, gpeak),
        "gemm2": stage_entry(stage_ms["gemm2"], g2_flop, g2_bytes, gpeak),
        "combine": stage_entry(stage_ms["combine"], 0.0, comb_bytes, declared="hbm"),
    }
    for n, b in (("gemm1_swiglu", g1_bytes), ("gemm2", g2_bytes)):
        stages[n]["hbm_gbs"] = gb(b, stages[n]["ms"])
    if comb_cold_ms is not None:
        stages["combine"]["mall_flushed"] = dict(ms=round(comb_cold_ms, 5), achieved=round(gb(comb_bytes, comb_cold_ms), 2),
                                                 frac=round(gb(comb_bytes, comb_cold_ms) / PEAK_HBM_GBS, 4))
    if gather:
        stages["permute"]["note"] = ("the sorted copy is never written: GEMM 1 gathers the x rows, so this stage "
                                     "moves index bytes only and its HBM fraction is not the permute target")
    if mx:
        stages["permute"]["rows"] = "index only; GEMM1 gathers the quantized x rows"
        stages["quantize_x"] = stage_entry(stage_ms["quantize_x"], 0.0, qx_bytes, declared="hbm")
    if bwd:
        wbytes_i, wbytes_o = e_nz * emb * 2 * mlp * 2, e_nz * mlp * emb * 2
        stages["combine_bwd"] = stage_entry(stage_ms["combine_bwd"], 0.0,
                                            T * emb * 2 + 2 * S * emb * 2 + 4 * S + 4 * S + 4 * S)
        stages["wgrad_dwo"] = stage_entry(stage_ms["wgrad_dwo"], 2.0 * S * mlp * emb,
                                          S * mlp * 2 + S * emb * 2 + E * mlp * emb * 2)
        if remat:
            stages["recompute_h"] = stage_entry(stage_ms["recompute_h"], g1_flop,
                                                S * emb * 2 + wbytes_i + S * mlp * 2 + S * 2 * mlp * 4)
        stages["gemm_dh"] = stage_entry(stage_ms["gemm_dh"], 2.0 * S * emb * mlp,
                                        T * emb * 2 + wbytes_o + S * 2 * mlp * 4 + S * 2 * mlp * 2 + 4 * S)
        stages["wgrad_dwi"] = stage_entry(stage_ms["wgrad_dwi"], 4.0 * S * emb * mlp,
                                          S * emb * 2 + S * 2 * mlp * 2 + E * emb * 2 * mlp * 2)
        stages["gemm_dxs"] = stage_entry(stage_ms["gemm_dxs"], 4.0 * S * emb * mlp,
                                         S * 2 * mlp * 2 + wbytes_i + S * emb * 2)
        stages["permute_bwd"] = stage_entry(stage_ms["permute_bwd"], 0.0, S * emb * 2 + 4 * S + T * emb * 2)
    if router_bwd:
        # x read once, dx read and written, Wr read (fp32), dWr written, per-slot index/weight/gradient reads
        rb_bytes = 3 * T * emb * 2 + 2 * emb * E * 4 + (4 + 4 + 4 + 4) * S
        stages["route_bwd"] = dict(stage_entry(stage_ms["route_bwd"], 0.0, rb_bytes, declared="hbm"),
                                   fp32_flop=4.0 * S * emb)
    fwd_flop = 6.0 * S * emb * mlp  # active-expert FLOPs of the two forward GEMMs
    gemm_ms = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]
    # the step at its roofline: the sum of the stages' floors
    floor_ms = sum(v["ms"] * v["frac"] for v in stages.values())
    return dict(wl=wl, inp=inp, ms_step=ms_step, tokens_per_s=T / (ms_step * 1e-3), stage_ms=stage_ms,
                stages=stages, fused_ms=fused_ms, bwd_fused_ms=bwd_fused_ms, graph_ms=graph_ms, gemm_ms=gemm_ms, gather=gather,
                layer_tflops=tf(fwd_flop * (3 if bwd else 1), ms_step),
                gemm_stage_tflops=tf(fwd_flop, gemm_ms), gemm_stage_frac=tf(fwd_flop, gemm_ms) / gpeak,
                floor_ms=floor_ms, e_nz=e_nz, g1_flop=g1_flop, gpeak=gpeak, router_bwd=router_bwd,
                saved_bytes=sum(v.numel() * v.element_size() for v in saved.values() if v is not None) if bwd
                else None)


def vendor_dense_gemm(wl, dev, iters=10):
    """Yardstick, not part of the step: the vendor library's dense bf16 GEMM (hipBLASLt through
    torch.matmul, contiguous 2-D operands) of the same total size and FLOPs as each grouped GEMM,
    [S, emb] x [emb, 2 mlp] and [S, mlp] x [mlp, emb], without SwiGLU or ragged groups."""
    import torch

    S = wl.T * wl.k
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    out = {"library": "hipBLASLt via torch.matmul (dense bf16, fp32 accumulate)",
           "note": "the same FLOPs as the grouped GEMM, as one dense GEMM; context for the roofline fraction"}
    for name, (m, kk, n) in (("gemm1", (S, wl.emb, 2 * wl.mlp)), ("gemm2", (S, wl.mlp, wl.emb))):
        a = torch.randn((m, kk), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = (torch.randn((kk, n), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        c = torch.empty((m, n), device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(iters):
            torch.matmul(a, b, out=c)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / iters
        flop = 2.0 * m * kk * n
        out[name] = {"m_k_n": [m, kk, n], "ms": round(ms, 5), "tflops": round(tf(flop, ms), 1),
                     "frac": round(tf(flop, ms) / PEAK_BF16_TFLOPS, 4)}
        del a, b, c
        torch.cuda.empty_cache()
    return out


def _round(d):
    return {k_: ({kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 if isinstance(v, dict) else (round(v, 5) if isinstance(v, float) else v)) for k_, v in d.items()}


def config_summary(r, steps, bwd):
    wl = r["wl"]
    return {
        "T": wl.T, "emb": wl.emb, "mlp": wl.mlp, "E": wl.E, "k": wl.k,
        "pass": "forward+backward" if bwd else "forward", "steps": steps,
        "ms_per_step": round(r["ms_step"], 4), "latency_us": round(r["ms_step"] * 1e3, 1),
        "tokens_per_s": round(r["tokens_per_s"], 1),
        "layer_tflops": round(r["layer_tflops"], 2),
        "gemm_stage_frac_of_mfma_peak": round(r["gemm_stage_frac"], 4),
        "roofline_floor_ms": round(r["floor_ms"], 4),
        "frac_of_roofline_floor": round(r["floor_ms"] / r["ms_step"], 4),
        "fused_entry_ms": None if r["fused_ms"] is None else round(r["fused_ms"], 4),
        "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 4),
        "bwd_fused_entry_ms": None if r["bwd_fused_ms"] is None else round(r["bwd_fused_ms"], 4),
        "stages": {n: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()
                       if kk in ("ms", "bound", "achieved", "unit", "frac")} for n, v in r["stages"].items()},
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this MoE FFN build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    bwd = args.backward
    remat = bwd and args.recompute_h
    mx = args.mxfp8 and not bwd
    r = measure(wl, dev, args.steps, args.warmup, bwd=bwd, remat=remat, mx=mx, flush_combine=not bwd)
    stages = r["stages"]

    # dominant kernel: grouped GEMM 1 (prefused wi + SwiGLU epilogue)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            # counters of the training step are filed under "<workload>:backward"; its GEMM 1 is the
            # plain-row kernel, the inference forward's the row-gather one
            key = args.workload + (":backward" if bwd else "")
            ent = None if mx else tr.get(key, {}).get("gemm1_swiglu")
            if ent and ent.get("source_sha") == source_hash(GEMM_SRC):
                traffic = ent["bytes_per_launch"]
        except Exception:
            traffic = None
    g1 = stages["gemm1_swiglu"]
    kname = ("mx_gemm_kernel<SWIGLU> (MXFP8 grouped GEMM 1 on prefused wi)" if mx else
             "gemm_kernel<NN,SWIGLU%s> (grouped GEMM 1 on prefused wi)" % (", row gather" if r["gather"] else ""))
    roofline = {"bound": g1["bound"], "kernel": kname,
                "achieved": round(g1["achieved"], 2), "peak": g1["peak"], "unit": g1["unit"],
                "frac": round(g1["frac"], 4), "traffic": traffic,
                "per_launch_flop": r["g1_flop"], "avg_launch_ms": round(g1["ms"], 5)}

    vendor = None
    if not (mx or bwd or args.no_vendor_yardstick):
        vendor = vendor_dense_gemm(wl, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(r["inp"], wl, args.cpu_seconds)
    del r["inp"]

    configs = None
    if not args.no_configs:
        configs = {}
        torch.cuda.empty_cache()
        for name, cbwd, csteps in CONFIGS:
            if name == args.workload:
                continue
            cr = measure(workloads.WORKLOADS[name], dev, csteps, 3, bwd=cbwd)
            del cr["inp"]
            configs[name] = config_summary(cr, csteps, cbwd)
            del cr
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "emb": wl.emb, "mlp": wl.mlp, "E": wl.E, "k": wl.k,
                   "pass": "forward+backward" if bwd else "forward", "router_backward": r["router_bwd"],
                   "recompute_h": remat, "gemm_operands": "mxfp8 (e4m3, e8m0 per 32)" if mx else "bf16",
                   "parallelism": "none (1 GPU)"},
        "layer_tflops": round(r["layer_tflops"], 2),
        "gemm_stage_tflops": round(r["gemm_stage_tflops"], 2),
        "gemm_stage_frac": round(r["gemm_stage_frac"], 4),
        "fused_entry_ms": None if r["fused_ms"] is None else round(r["fused_ms"], 4),
        "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 4),
        "bwd_fused_entry_ms": None if r["bwd_fused_ms"] is None else round(r["bwd_fused_ms"], 4),
        # activations kept from the forward for the backward (the saved set)
        "saved_bytes": r["saved_bytes"],
        "stages": {k_: _round(v) for k_, v in stages.items()},
        "roofline": roofline,
        "vendor_dense_gemm": vendor,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    if args.stage_json:
        json.dump(line, open(args.stage_json, "w"), indent=1)
    print(json.dumps(line), flush=True)


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, wl, target_s: float):
    """The oracle as it stands, on a bounded token sample of the same workload, on the host cores."""
    import numpy as np

    import oracle
    import workloads

    threads = oracle.default_threads()
    xb = workloads.bf16_bits(inp["x"])
    wib = workloads.bf16_bits(inp["wi"])
    wob = workloads.bf16_bits(inp["wo"])
    wr = None if inp["wr"] is None else inp["wr"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    logits = None if inp["logits_in"] is None else inp["logits_in"].cpu().numpy()
    rng = np.random.default_rng(0)

    def run(n):
        toks = np.sort(rng.choice(wl.T, n, replace=False))
        t0 = time.perf_counter()
        idx, w, _ = oracle.route(xb[toks], wr, bias, wl.k, logits_in=None if logits is None else logits[toks],
                                 threads=threads)
        oracle.ffn_fwd_tokens(xb[toks], idx, w, wib, wob, threads=threads)
        return time.perf_counter() - t0

    n = threads
    dt = run(n)
    n = int(max(threads, min(wl.T, n * target_s / max(dt, 1e-3))))
    dt = run(n)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": avail, "cpu_model": _cpu_model(),
            "threads_note": "one oracle thread per host CPU, capped at 16 (the host share of one GPU on the "
                            "measurement machine)",
            "sample": f"{n} of {wl.T} tokens of {wl.name}: fp32 router + top-k + per-token FFN forward "
                      f"(fp32 accumulate), {dt:.1f} s on {threads} threads"}


if __name__ == "__main__":
    main()
