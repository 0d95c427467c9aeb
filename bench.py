"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gemma4_class]
                    [--backward [--recompute-h] | --mxfp8] [--no-cpu-baseline] [--stage-json PATH]

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
the layer backward (combine-bwd, NT GEMM + SwiGLU-bwd, NT GEMM, permute-bwd,
wgrad x2) and, where the router is learned, the router backward (logit
gradients from dtopk_w, dWr, and dx += dlogits . Wr^T onto the layer's dx).
With --mxfp8 the forward runs its grouped GEMMs on MXFP8 operands: each token
row of x is quantized once and GEMM 1 reads the codes through sorted_slot,
GEMM 1's SwiGLU epilogue writes its output as MXFP8 for GEMM 2, and the
expert weights are quantized beforehand (weight preparation, outside the
timed step).
With --recompute-h the forward keeps no fp32 gate/up values and the backward
recomputes them with one more GEMM1 (the saved bytes are reported).
"""
from __future__ import annotations

import argparse
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--stage-json", default=None, help="also write per-stage details to this file")
    return ap.parse_args()


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this MoE FFN build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_ffn_group_amd as moe
    import workloads
    from mixture_experts_ffn_group_amd import _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.WORKLOADS[args.workload]
    T, emb, mlp, E, k, S = wl.T, wl.emb, wl.mlp, wl.E, wl.k, wl.S
    inp = workloads.make_inputs(wl, device=dev)
    x, wi, wo, wr, bias, logits = inp["x"], inp["wi"], inp["wo"], inp["wr"], inp["bias"], inp["logits_in"]
    moe.query_support(T, emb, mlp, E, k)
    stream = torch.cuda.current_stream(dev)

    # buffers (allocated once, outside the timed region)
    bwd = args.backward
    remat = bwd and args.recompute_h
    saved = moe.alloc_saved(T, emb, mlp, E, k, dev, keep_h=not remat)
    y = torch.empty((T, emb), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.workspace_bytes(T, emb, mlp, E, k), dtype=torch.uint8, device=dev)
    pws = torch.empty(max(16, int(_lib.lib().moe_permute_workspace_bytes(
        __import__("ctypes").byref(_lib.shape(T, emb, mlp, E, k))))), dtype=torch.uint8, device=dev)
    if bwd:
        dy = inp["dy"]
        bws = torch.empty(moe.workspace_bytes(T, emb, mlp, E, k, backward=True, recompute_h=remat),
                          dtype=torch.uint8, device=dev)
        grads = dict(dx=torch.empty((T, emb), dtype=torch.bfloat16, device=dev),
                     dwi=torch.empty_like(wi), dwo=torch.empty_like(wo),
                     dtopk_w=torch.empty((T, k), dtype=torch.float32, device=dev))
    router_bwd = bwd and wr is not None
    if router_bwd:
        rbws = torch.empty(max(16, int(_lib.lib().moe_route_bwd_workspace_bytes(
            __import__("ctypes").byref(_lib.shape(T, emb, mlp, E, k))))), dtype=torch.uint8, device=dev)
        grads["dwr"] = torch.empty((emb, E), dtype=torch.float32, device=dev)
        grads["dbias"] = torch.empty(E, dtype=torch.float32, device=dev) if bias is not None else None

    import ctypes as C
    L = _lib.lib()
    shp = _lib.shape(T, emb, mlp, E, k)
    P = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    st = C.c_void_p(stream.cuda_stream)
    sv = saved

    # Inference (forward only) runs the path moe_ffn_fwd takes without a saved set: the permute builds
    # the index only and GEMM1 gathers the x rows through sorted_slot. With --backward the forward
    # materialises xs and h, which the backward reads.
    gather = not bwd
    rows = _lib.MoeGemmRows(P(sv["sorted_slot"]), S, k, None) if gather else None

    mx = args.mxfp8 and not bwd
    if mx:
        # MXFP8 operands: weights quantized once (weight preparation, outside the timed step), activations in it
        wiq, wis = moe.mx_quantize_weight(wi)       # [E, 2mlp, emb], [E, emb/64, 2mlp, 4]
        woq, wos = moe.mx_quantize_weight(wo)       # [E, emb, mlp], [E, mlp/64, emb, 4]
        xq = torch.empty((T, emb), dtype=torch.uint8, device=dev)   # token rows, read by GEMM 1 through sorted_slot
        xqs = torch.empty((emb // 64, T, 4), dtype=torch.uint8, device=dev)
        aq = torch.empty((S, mlp), dtype=torch.uint8, device=dev)
        aqs = torch.empty((mlp // 64, S, 4), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def stage_calls():
        """The forward (and optional backward) as separate library calls, in moe_ffn_fwd order."""
        if mx:
            return [
                ("route", lambda: L.moe_route(C.byref(shp), None if logits is not None else P(x), P(wr), P(bias),
                                              P(logits), P(sv["topk_idx"]), P(sv["topk_w"]), st)),
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
                ("combine", lambda: L.moe_combine(C.byref(shp), P(sv["o"]), P(sv["slot_row"]), P(sv["topk_w"]),
                                                  P(y), st)),
            ]
        calls = [
            ("route", lambda: L.moe_route(C.byref(shp), None if logits is not None else P(x), P(wr), P(bias),
                                          P(logits), P(sv["topk_idx"]), P(sv["topk_w"]), st)),
            ("permute", lambda: L.moe_permute(C.byref(shp), P(x), P(sv["topk_idx"]), P(sv["group_sizes"]),
                                              P(sv["group_offsets"]), P(sv["sorted_slot"]), P(sv["slot_row"]),
                                              None if gather else P(sv["xs"]), P(pws), pws.numel(), st)),
            ("gemm1_swiglu", lambda: L.moe_grouped_gemm(0, 1, P(x) if gather else P(sv["xs"]), P(wi), None,
                                                        P(sv["h"]) if bwd else None, P(sv["group_offsets"]), E, S,
                                                        emb, 2 * mlp, C.byref(rows) if gather else None,
                                                        P(sv["a"]), st)),
            ("gemm2", lambda: L.moe_grouped_gemm(0, 0, P(sv["a"]), P(wo), None, None, P(sv["group_offsets"]), E, S,
                                                 mlp, emb, None, P(sv["o"]), st)),
            ("combine", lambda: L.moe_combine(C.byref(shp), P(sv["o"]), P(sv["slot_row"]), P(sv["topk_w"]), P(y),
                                              st)),
        ]
        if bwd:
            calls.append(("backward", lambda: L.moe_ffn_bwd(C.byref(shp), P(dy), C.byref(moe._saved_struct(sv)),
                                                            P(wi), P(wo), P(grads["dx"]), P(grads["dwi"]),
                                                            P(grads["dwo"]), P(grads["dtopk_w"]), P(bws), bws.numel(),
                                                            st)))
        if router_bwd:
            calls.append(("route_bwd", lambda: L.moe_route_bwd(C.byref(shp), P(x), P(wr), P(sv["topk_idx"]),
                                                               P(sv["topk_w"]), P(grads["dtopk_w"]),
                                                               P(sv["sorted_slot"]), P(sv["group_offsets"]),
                                                               P(grads["dwr"]), P(grads["dbias"]), P(grads["dx"]),
                                                               P(rbws), rbws.numel(), st)))
        return calls

    calls = stage_calls()

    def run_step(events=None):
        for i, (name, f) in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            rc = f()
            if rc != 0:
                raise _lib.MoeError(rc, name, L.moe_last_error_detail().decode())
        if events is not None:
            events[len(calls)].record(stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                for i, (name, _) in enumerate(calls)}

    # the fused entry point over the same buffers, as a cross-check of the staged timing
    fused_ms = None
    if mx:
        wq = dict(wi_codes=wiq, wi_scales=wis, wo_codes=woq, wo_scales=wos, mlp=mlp)
        mws = torch.empty(int(L.moe_workspace_bytes_mx(C.byref(shp))), dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            moe.ffn_fwd_mx(x, wq, k, wr=wr, bias=bias, logits=logits, workspace=mws, out=y)
        e0.record(stream)
        for _ in range(args.steps):
            moe.ffn_fwd_mx(x, wq, k, wr=wr, bias=bias, logits=logits, workspace=mws, out=y)
        e1.record(stream)
        torch.cuda.synchronize()
        fused_ms = e0.elapsed_time(e1) / args.steps
    if not bwd and not mx:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            moe.ffn_fwd(x, wi, wo, k, wr=wr, bias=bias, logits=logits, workspace=ws, out=y)
        e0.record(stream)
        for _ in range(args.steps):
            moe.ffn_fwd(x, wi, wo, k, wr=wr, bias=bias, logits=logits, workspace=ws, out=y)
        e1.record(stream)
        torch.cuda.synchronize()
        fused_ms = e0.elapsed_time(e1) / args.steps

    # The combine again, alone, with the 256 MB MALL (Infinity Cache) flushed before each launch: in the step
    # it reads o right after GEMM 2 wrote it, so part of o may still be in the MALL there. The flush writes a
    # 512 MB buffer and then reads it back, so that its own dirty lines are written back before the launch.
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
    ms_step = wall * 1e3 / args.steps
    tokens_per_s = T / (ms_step * 1e-3)
    fwd_flop = 6.0 * S * emb * mlp              # active-expert FLOPs of the two GEMMs
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

    def tf(flop, ms):
        return flop / (ms * 1e-3) / 1e12

    def gb(b, ms):
        return b / (ms * 1e-3) / 1e9

    stages = {
        "route": dict(ms=stage_ms["route"], bound="mfma" if route_flop else "hbm",
                      achieved=tf(route_flop, stage_ms["route"]) if route_flop else gb(route_bytes, stage_ms["route"]),
                      peak=PEAK_FP32_MFMA_TFLOPS if route_flop else PEAK_HBM_GBS,
                      unit="TFLOP/s" if route_flop else "GB/s"),
        "permute": dict(ms=stage_ms["permute"], bound="hbm", achieved=gb(perm_bytes, stage_ms["permute"]),
                        peak=PEAK_HBM_GBS, unit="GB/s", bytes=perm_bytes,
                        rows="index only; GEMM1 gathers the x rows" if gather else "rows copied to xs"),
        "gemm1_swiglu": dict(ms=stage_ms["gemm1_swiglu"], bound="mfma",
                             achieved=tf(g1_flop, stage_ms["gemm1_swiglu"]), peak=gpeak, unit="TFLOP/s",
                             flop=g1_flop, bytes=g1_bytes, hbm_gbs=gb(g1_bytes, stage_ms["gemm1_swiglu"])),
        "gemm2": dict(ms=stage_ms["gemm2"], bound="mfma", achieved=tf(g2_flop, stage_ms["gemm2"]),
                      peak=gpeak, unit="TFLOP/s", flop=g2_flop, bytes=g2_bytes,
                      hbm_gbs=gb(g2_bytes, stage_ms["gemm2"])),
        "combine": dict(ms=stage_ms["combine"], bound="hbm", achieved=gb(comb_bytes, stage_ms["combine"]),
                        peak=PEAK_HBM_GBS, unit="GB/s", bytes=comb_bytes,
                        mall_flushed=dict(ms=round(comb_cold_ms, 5), achieved=round(gb(comb_bytes, comb_cold_ms), 2),
                                          frac=round(gb(comb_bytes, comb_cold_ms) / PEAK_HBM_GBS, 4))),
    }
    if mx:
        stages["permute"]["rows"] = "index only; GEMM1 gathers the quantized x rows"
        stages["quantize_x"] = dict(ms=stage_ms["quantize_x"], bound="hbm", achieved=gb(qx_bytes, stage_ms["quantize_x"]),
                                    peak=PEAK_HBM_GBS, unit="GB/s", bytes=qx_bytes)
    if bwd:
        stages["backward"] = dict(ms=stage_ms["backward"], bound="mfma",
                                  achieved=tf(12.0 * S * emb * mlp, stage_ms["backward"]), peak=PEAK_BF16_TFLOPS,
                                  unit="TFLOP/s")
    if router_bwd:
        # x read once, dx read and written, Wr read (fp32), dWr written, per-slot index/weight/gradient reads
        rb_bytes = 3 * T * emb * 2 + 2 * emb * E * 4 + (4 + 4 + 4 + 4) * S
        stages["route_bwd"] = dict(ms=stage_ms["route_bwd"], bound="hbm", achieved=gb(rb_bytes, stage_ms["route_bwd"]),
                                   peak=PEAK_HBM_GBS, unit="GB/s", bytes=rb_bytes,
                                   fp32_flop=4.0 * S * emb)
    for v in stages.values():
        v["frac"] = v["achieved"] / v["peak"]
    gemm_ms = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]

    # dominant kernel: grouped GEMM 1 (prefused wi + SwiGLU epilogue)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ent = None if mx else tr.get(args.workload, {}).get("gemm1_swiglu")
            if ent and ent.get("source_sha") == source_hash(GEMM_SRC):
                traffic = ent["bytes_per_launch"]
        except Exception:
            traffic = None
    g1 = stages["gemm1_swiglu"]
    kname = ("mx_gemm_kernel<SWIGLU> (MXFP8 grouped GEMM 1 on prefused wi)" if mx else
             "gemm_kernel<NN,SWIGLU%s> (grouped GEMM 1 on prefused wi)" % (", row gather" if gather else ""))
    roofline = {"bound": "mfma", "kernel": kname,
                "achieved": round(g1["achieved"], 2), "peak": gpeak, "unit": "TFLOP/s",
                "frac": round(g1["frac"], 4), "traffic": traffic,
                "per_launch_flop": g1_flop, "avg_launch_ms": round(g1["ms"], 5)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wl, args.cpu_seconds)

    line = {
        "metric": "MoE FFN layer tokens/s + achieved bf16 MFMA TFLOP/s, 128 experts top-8",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "emb": emb, "mlp": mlp, "E": E, "k": k,
                   "pass": "forward+backward" if bwd else "forward", "router_backward": router_bwd,
                   "recompute_h": remat, "gemm_operands": "mxfp8 (e4m3, e8m0 per 32)" if mx else "bf16",
                   "parallelism": "none (1 GPU)"},
        "layer_tflops": round(tf(fwd_flop * (3 if bwd else 1), ms_step), 2),
        "gemm_stage_tflops": round(tf(fwd_flop, gemm_ms), 2),
        "gemm_stage_frac": round(tf(fwd_flop, gemm_ms) / gpeak, 4),
        "fused_entry_ms": None if fused_ms is None else round(fused_ms, 4),
        # activations kept from the forward for the backward (the saved set)
        "saved_bytes": sum(v.numel() * v.element_size() for v in saved.values() if v is not None) if bwd else None,
        "stages": {k_: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k_, v in stages.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.stage_json:
        json.dump(line, open(args.stage_json, "w"), indent=1)
    print(json.dumps(line), flush=True)


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
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.T} tokens of {wl.name}: fp32 router + top-k + per-token FFN forward "
                      f"(fp32 accumulate), {dt:.1f} s on {threads} threads"}


if __name__ == "__main__":
    main()
