"""Benchmark of one routed-MoE layer (router -> align -> up+SwiGLU -> down -> finalize) on
one MI355X, through the C ABI.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload decode_m8]
                    [--no-sweep] [--no-cpu-baseline] [--no-mx]

Prints ONE JSON line.  A step is one moe_forward call (all five kernels) over resident
inputs of the workload; K steps are timed between two synchronisations (wall clock and
HIP events on the launch stream, the larger is used).  A second pass of K steps records
six HIP events per step around the five kernels for the per-kernel durations (an event
between two kernels adds a few microseconds of idle, so that pass is not the headline).
`value` is tokens/s of the headline workload (decode, M=8); `sweep` holds the same
measurement at M=128, 512 and 2048 on the same weights, each with its own `roofline`.

`roofline` is for the dominant kernel (the grouped up-GEMM + SwiGLU, which streams W13):
algorithmic bytes per launch / its average duration from the HIP events, against the
8 TB/s HBM peak, with the MFMA rate of the same launch against the 2.5 PFLOP/s bf16 dense
peak beside it; `traffic` is the HBM bytes that rocprofv3's FETCH_SIZE + WRITE_SIZE
counters read for that kernel (profiles/traffic_*.json, null once the kernel source has
changed since).  `measured_read_peak` is the best of the read probes over the resident
W13 (probe/read_bw.hip): a plain nontemporal vector-load pass, and the tiled GEMMs' own
copy path (nontemporal global_load_lds whole-line copies into LDS rings, 256-row items on
one workgroup per CU and 128-row items on two or three).
`cpu_baseline` is the CPU oracle timed on the GPU run's own inputs (copied to the host).
`mxfp8_decode` times the same layer with the expert weights quantized to MXFP8
(moe_forward_mx); it is a separate measurement, not the headline, whose weights are bf16.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "MoE-layer tokens/s and µs/layer at M=8/128/2048; % HBM or MFMA roofline"
STAGES = ("route", "align", "up", "down", "finalize")
PROFILES = os.path.join(ROOT, "profiles")
SWEEP = ("batch_m128", "batch_m512", "prefill_m2048")


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def weight_bytes_per_value(fmt):
    """bf16: 2 bytes; MXFP8: one E4M3 byte plus one scale byte per 32 values; MXFP4: half a
    byte per E2M1 code plus one scale byte per 32 values."""
    return {"bf16": 2, "mx8": 1 + 1 / 32, "mx4": 0.5 + 1 / 32}[fmt]


def layer_bytes(cfg, M, touched, fmt="bf16"):
    """Algorithmic HBM bytes of one layer: touched experts' W13+W2, the router weight,
    x, residual and out rows, and the norm weight."""
    per_expert = 3 * cfg.I * cfg.H * weight_bytes_per_value(fmt)
    return int(touched * per_expert) + cfg.E * cfg.H * 2 + 3 * M * cfg.H * 2 + cfg.H * 2


def up_bytes(cfg, M, touched, fmt="bf16"):
    """Algorithmic bytes of the up kernel: W13 of every touched expert, each token's x
    row once, and one bf16 act row per (token, pick)."""
    return (int(touched * 2 * cfg.I * cfg.H * weight_bytes_per_value(fmt)) + M * cfg.H * 2
            + M * cfg.top_k * cfg.I * 2)


def down_bytes(cfg, M, touched, fmt="bf16"):
    """Algorithmic bytes of the down kernel: W2 of every touched expert, one bf16 act row
    read and one bf16 y row written per (token, pick)."""
    return (int(touched * cfg.H * cfg.I * weight_bytes_per_value(fmt))
            + M * cfg.top_k * (cfg.I + cfg.H) * 2)


def layer_flops(cfg, M):
    return 2 * M * cfg.E * cfg.H + 6 * M * cfg.top_k * cfg.H * cfg.I


def up_flops(cfg, M):
    return 4 * M * cfg.top_k * cfg.H * cfg.I


def down_flops(cfg, M):
    return 2 * M * cfg.top_k * cfg.I * cfg.H


def run_workload(B, mi, torch, cfg, weights, steps, warmup, dev, mx=None, prepared=None,
                 mx4=None, mxp=None):
    """Times moe_forward (bf16 experts), moe_forward_mx when `mx` holds the MXFP8
    (w13 codes, w13 scales, w2 codes, w2 scales), moe_forward_prepared when `prepared`
    holds the prepared (w13, w2) stacks, moe_forward_mx4 when `mx4` holds the MXFP4
    panels, or moe_forward_mx_prepared when `mxp` holds the MXFP8 panels (each as w13
    codes, w13 scales, w2 codes, w2 scales)."""
    L = mi.make_layer(cfg, device=dev, seed=0, with_experts=False)
    L.update(weights)
    M, H, E, I, k, blk = cfg.M, cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(M, H, E, I, k, blk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        if mxp is not None:
            B.moe_forward_mx_prepared(L["x"], L["router_w"], L["router_bias"], *mxp, I,
                                      L["residual"], L["norm_w"], L["eps"], k, blk, out, ws,
                                      topk_ids_out=ids, stage_events=events, stream=stream)
        elif mx4 is not None:
            B.moe_forward_mx4(L["x"], L["router_w"], L["router_bias"], *mx4, I, L["residual"],
                              L["norm_w"], L["eps"], k, blk, out, ws, topk_ids_out=ids,
                              stage_events=events, stream=stream)
        elif prepared is not None:
            B.moe_forward_prepared(L["x"], L["router_w"], L["router_bias"], prepared[0],
                                   prepared[1], I, L["residual"], L["norm_w"], L["eps"], k, blk,
                                   out, ws, topk_ids_out=ids, stage_events=events, stream=stream)
        elif mx is None:
            B.moe_forward(L["x"], L["router_w"], L["router_bias"], L["w13"], L["w2"],
                          L["residual"], L["norm_w"], L["eps"], k, blk, out, ws,
                          topk_ids_out=ids, stage_events=events, stream=stream)
        else:
            B.moe_forward_mx(L["x"], L["router_w"], L["router_bias"], *mx, L["residual"],
                             L["norm_w"], L["eps"], k, blk, out, ws, topk_ids_out=ids,
                             stage_events=events, stream=stream)

    for _ in range(warmup):
        step()
    # timed region: K back-to-back layers, nothing recorded between the kernels
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge = [B.HipEvent(), B.HipEvent()]
    edge[0].record(stream)
    for _ in range(steps):
        step()
    edge[1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    span_ms = B.HipEvent.elapsed_ms(edge[0], edge[1]) / steps
    # per-kernel breakdown: the same K layers again with six HIP events around the five
    # kernels of every layer, recorded on the launch stream
    events = [[B.HipEvent() for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        step(events[s])
    torch.cuda.synchronize()
    stage_ms = {name: sum(B.HipEvent.elapsed_ms(ev[i], ev[i + 1]) for ev in events) / steps
                for i, name in enumerate(STAGES)}
    # per-layer distribution of that pass (first to last event of each layer)
    per_layer = sorted(B.HipEvent.elapsed_ms(ev[0], ev[-1]) * 1e3 for ev in events)

    def pct(q):
        x = q * (len(per_layer) - 1)
        lo = int(x)
        hi = min(lo + 1, len(per_layer) - 1)
        return per_layer[lo] + (per_layer[hi] - per_layer[lo]) * (x - lo)
    ms = max(wall_ms, span_ms)
    touched = int(torch.unique(ids).numel())
    counts = torch.bincount(ids.flatten().long(), minlength=E)
    fmt = "mx8" if (mx is not None or mxp is not None) else "mx4" if mx4 is not None else "bf16"
    lb = layer_bytes(cfg, M, touched, fmt)
    ub = up_bytes(cfg, M, touched, fmt)
    db = down_bytes(cfg, M, touched, fmt)
    stages = {n: round(v * 1e3, 2) for n, v in stage_ms.items()}
    self_routed = (mx is None and prepared is None and mx4 is None and mxp is None
                   and B.moe_forward_self_routes(M, E, k, I))
    if self_routed:
        # the up GEMM builds the plan: no align kernel runs, the event pair encloses none
        stages["align"] = None
    return {
        "M": M, "ms_per_step": ms, "us_per_layer": ms * 1e3, "tokens_per_s": M / (ms / 1e3),
        "wall_ms": wall_ms, "event_span_ms": span_ms, "stages_us": stages,
        "layer_us_p10_p50_p90": [round(pct(0.1), 2), round(pct(0.5), 2), round(pct(0.9), 2)],
        "align": "fused into the up GEMM (self-routing)" if self_routed else "align kernel",
        "touched_experts": touched, "max_expert_count": int(counts.max().item()),
        "plan_rows": int(sum(((c + blk - 1) // blk) * blk for c in counts.tolist())),
        "layer_bytes": lb, "layer_gbs": lb / (ms / 1e3) / 1e9,
        "layer_hbm_frac": lb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac": layer_flops(cfg, M) / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        "up_bytes": ub, "up_us": stage_ms["up"] * 1e3,
        "up_gbs": ub / (stage_ms["up"] / 1e3) / 1e9,
        "up_tflops": up_flops(cfg, M) / (stage_ms["up"] / 1e3) / 1e12,
        "down_bytes": db, "down_us": stage_ms["down"] * 1e3,
        "down_gbs": db / (stage_ms["down"] / 1e3) / 1e9,
        "down_tflops": down_flops(cfg, M) / (stage_ms["down"] / 1e3) / 1e12,
    }


def up_kernel_name(B, cfg, mx=False):
    M, E, k, I = cfg.M, cfg.E, cfg.top_k, cfg.I
    if mx:
        rows = B.moe_gemm_tile_rows_mx(M, E, k, I)
        return (f"expert_tiled_mx_kernel<{rows}, ...>" if rows == 128
                else f"expert_mx_decode_kernel<true> ({rows}-row tiles)")
    rows = B.moe_gemm_tile_rows(M, E, k, I)
    if B.moe_forward_self_routes(M, E, k, I):
        return f"expert_up_selfroute_kernel<{rows}, ...> (align fused in)"
    if rows == 16:
        return "expert_up_stream_kernel"
    return f"expert_tiled ({rows}-row tiles, up)"


def _tile_rows(kernel: str):
    """Token-tile height named in a kernel label ("...<128, ..." or "(64-row tiles"), or None."""
    m = re.search(r"<(\d+),|\((\d+)-row", kernel)
    return None if m is None else int(m.group(1) or m.group(2))


def load_profile(name: str, workload: str, kernel: str):
    """A counter summary under profiles/ (FETCH_SIZE / WRITE_SIZE, MFMA busy), or None when
    it is missing, was taken on another workload or another tile height than `kernel` runs
    with, or the kernel source changed since."""
    try:
        with open(os.path.join(PROFILES, name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or _tile_rows(t.get("kernel", "")) != _tile_rows(kernel):
        return None
    src = os.path.join(ROOT, "prefill_sigmoid_router_amd", "csrc", t.get("source_file", ""))
    if not os.path.isfile(src) or t.get("source_sha256_16") != source_hash(src):
        return None
    return t


def roofline(res, kernel, read_peak, prof):
    """The roofline object of a leg: the up GEMM's algorithmic bytes and flops over its
    average launch duration (HIP events on the launch stream)."""
    r = {
        "bound": "hbm", "kernel": f"{kernel} (grouped up-GEMM + SwiGLU)",
        "achieved": round(res["up_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(res["up_gbs"] / HBM_PEAK_GBS, 4),
        "traffic": None if prof is None else prof.get("traffic_gbs"),
        "traffic_bytes_per_launch": None if prof is None else prof.get("traffic_bytes_per_launch"),
        "algorithmic_bytes_per_launch": res["up_bytes"], "avg_launch_us": round(res["up_us"], 2),
        "mfma_achieved_tflops": round(res["up_tflops"], 1), "mfma_peak_tflops": BF16_PEAK_TFLOPS,
        "mfma_frac": round(res["up_tflops"] / BF16_PEAK_TFLOPS, 4),
        "down_gbs": round(res["down_gbs"], 1),
        "down_frac": round(res["down_gbs"] / HBM_PEAK_GBS, 4),
        "down_mfma_frac": round(res["down_tflops"] / BF16_PEAK_TFLOPS, 4),
    }
    if read_peak:
        r["measured_read_peak"] = round(read_peak, 1)
        r["frac_of_measured_read"] = round(res["up_gbs"] / read_peak, 4)
    if prof is not None and prof.get("mfma_busy_frac") is not None:
        r["mfma_busy_frac_counter"] = prof["mfma_busy_frac"]
    return r


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle on the GPU run's own inputs
# ---------------------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def _host_inputs(mi, cfg, weights, dev):
    """The GPU run's inputs of workload cfg, as host bit patterns."""
    L = mi.make_layer(cfg, device=dev, seed=0, with_experts=False)
    bits = mi.bf16_bits
    return {"x": bits(L["x"]), "residual": bits(L["residual"]),
            "router_w": bits(weights["router_w"]), "norm_w": bits(weights["norm_w"]),
            "bias": None if L["router_bias"] is None else L["router_bias"].cpu().numpy(),
            "eps": L["eps"]}


def cpu_decode(mi, weights, dev, runs=3):
    """The oracle's whole-layer forward (fp64 numpy, plan based) over all tokens of the
    decode workload, on the GPU's inputs and experts copied to the host; median of runs."""
    from oracle import moe_oracle as orc
    cfg = mi.CONFIGS["decode_m8"]
    h = _host_inputs(mi, cfg, weights, dev)
    ids, _, _ = orc.route(h["x"], h["router_w"], h["bias"], cfg.top_k)
    need = sorted(set(int(e) for e in ids.ravel()))
    w13 = {e: mi.bf16_bits(weights["w13"][e]) for e in need}       # copied before timing
    w2 = {e: mi.bf16_bits(weights["w2"][e]) for e in need}
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        orc.forward(h["x"], h["router_w"], h["bias"], w13, w2, h["residual"], h["norm_w"],
                    h["eps"], cfg.top_k, cfg.block)
        times.append(time.perf_counter() - t0)
    sec = sorted(times)[len(times) // 2]
    return sec, len(need), times


def cpu_sampled(mi, cfg, weights, dev, n_experts=16, seed=0):
    """The oracle's steps on the GPU's inputs of a larger workload, with the expert step on
    a bounded sample: route and align over every token, the up and down projections of the
    plan blocks of n_experts seeded experts (scaled to all touched experts by their share
    of plan blocks), the finalize over every token.  Returns the estimated seconds."""
    import numpy as np
    from oracle import moe_oracle as orc
    h = _host_inputs(mi, cfg, weights, dev)
    t0 = time.perf_counter()
    ids, w, _ = orc.route(h["x"], h["router_w"], h["bias"], cfg.top_k)
    sorted_ids, bexp, n_pad, counts, _ = orc.align(ids, cfg.E, cfg.block)
    t_plan = time.perf_counter() - t0
    touched = np.nonzero(counts)[0]
    pick = set(np.random.default_rng(seed).choice(touched, size=min(n_experts, len(touched)),
                                                  replace=False).tolist())
    x = orc.bf16_to_f64(h["x"])
    n = cfg.M * cfg.top_k
    blocks = [b for b in range(n_pad // cfg.block) if int(bexp[b]) in pick]
    w13 = {e: mi.bf16_bits(weights["w13"][e]) for e in pick}       # copied before timing
    w2 = {e: mi.bf16_bits(weights["w2"][e]) for e in pick}
    y = np.zeros((n, cfg.H))
    t0 = time.perf_counter()
    for b in blocks:
        e = int(bexp[b])
        rows = sorted_ids[b * cfg.block:(b + 1) * cfg.block]
        live = rows[rows < n]
        if live.size:
            act = orc.expert_swiglu(x[live // cfg.top_k], w13[e], cfg.I)
            y[live] = orc.expert_down(act, w2[e])
    t_exp = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.finalize(y, w, h["residual"], h["norm_w"], h["eps"])
    t_fin = time.perf_counter() - t0
    all_blocks = n_pad // cfg.block
    return t_plan + t_exp * all_blocks / max(1, len(blocks)) + t_fin, len(blocks), all_blocks


def cpu_baseline(mi, torch, weights, dev, sweep=True):
    cores = len(os.sched_getaffinity(0))
    blas = _blas_threads()
    sec, touched, times = cpu_decode(mi, weights, dev)
    cfg = mi.CONFIGS["decode_m8"]
    line = {
        "value": cfg.M / sec, "unit": "tokens/s", "cores": blas, "kind": "oracle",
        "sample": (f"decode_m8, the GPU run's own inputs and experts copied to the host: all "
                   f"{cfg.M} tokens through the oracle's whole layer (fp64 numpy, bf16 weights "
                   f"decoded inside the timed region), {touched} experts; median of "
                   f"{len(times)} runs = {sec:.2f} s"),
        "cpu_model": _cpu_model(), "host_cpus": cores, "blas_threads": blas,
    }
    if sweep:
        est = {}
        for name, runs in (("batch_m128", 3), ("batch_m512", 1), ("prefill_m2048", 1)):
            c = mi.CONFIGS[name]
            vals = [cpu_sampled(mi, c, weights, dev, seed=r) for r in range(runs)]
            s = sorted(v[0] for v in vals)[len(vals) // 2]
            est[name] = {"value": round(c.M / s, 3), "unit": "tokens/s", "seconds": round(s, 2),
                         "runs": runs,
                         "sample": (f"route, align and finalize over all {c.M} tokens; up and "
                                    f"down projections of the plan blocks of 16 seeded experts "
                                    f"({vals[0][1]} of {vals[0][2]} blocks), scaled to every "
                                    f"block")}
        line["sweep_estimates"] = est
    return line


# ---------------------------------------------------------------------------------------
# Read probes
# ---------------------------------------------------------------------------------------
def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "prefill_sigmoid_router_amd", "libmoe_probe.so"))
    lib.moe_probe_read.restype = ctypes.c_int
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.moe_probe_read_grid.restype = ctypes.c_int
    lib.moe_probe_read_lds.restype = ctypes.c_int
    lib.moe_probe_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    return lib


def _best_ms(torch, stream, once, reps):
    once()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        once()
        b.record(stream)
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


def read_probe_gbs(torch, dev, buf, reps=5):
    """Plain pass: coalesced nontemporal vector loads over `buf`, best of reps."""
    import ctypes
    lib = _probe_lib()
    n = buf.numel() * buf.element_size() // 16 * 16
    sink = torch.empty(lib.moe_probe_read_grid(), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def once():
        st = lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()), n,
                                ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"moe_probe_read failed with status {st}")

    return n / (_best_ms(torch, stream, once, reps) * 1e-3) / 1e9


def read_probe_lds_gbs(torch, dev, w13, reps=5):
    """The tiled up GEMMs' copy path over the W13 stack [E, 2I, H]: nontemporal
    global_load_lds whole-line copies in the kernels' XCD-aware item order, no arithmetic:
    items of 256 rows (128 gate + 128 up) on one 4-wave workgroup per CU through rings of
    3, 4 and 5 chunks of 32 KiB, and items of 128 rows on two or three workgroups per CU
    through rings of 3 or 4 chunks of 16 KiB; the best rate of each over reps passes."""
    import ctypes
    lib = _probe_lib()
    E, two_i, K = w13.shape
    cus = torch.cuda.get_device_properties(dev).multi_processor_count // 8 * 8
    sink = torch.empty(3 * cus, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    rates = {}
    for rows, stages, per_cu in ((256, 3, 1), (256, 4, 1), (256, 5, 1), (128, 3, 2),
                                 (128, 3, 3), (128, 4, 2)):
        def once():
            st = lib.moe_probe_read_lds(ctypes.c_void_p(w13.data_ptr()), E, two_i // 2, K, stages,
                                        rows, per_cu * cus, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError(f"moe_probe_read_lds failed with status {st}")

        rates[(rows, stages, per_cu)] = (w13.numel() * 2 /
                                         (_best_ms(torch, stream, once, reps) * 1e-3) / 1e9)
    return rates


def read_probes(torch, dev, w13):
    """Every read probe over `w13`, by name: GB/s."""
    out = {"plain_nontemporal_loads": read_probe_gbs(torch, dev, w13)}
    for (rows, stages, per_cu), g in read_probe_lds_gbs(torch, dev, w13).items():
        out[f"global_load_lds_nt_{rows}_rows_{stages}_stages_{per_cu}_per_cu"] = g
    return out


def _rounded(r):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_m8")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the legs with MXFP8 expert weights")
    ap.add_argument("--no-prepared", action="store_true",
                    help="skip the legs on prepared (fragment-panel) weights")
    ap.add_argument("--no-mx4", action="store_true",
                    help="skip the legs with MXFP4 expert weights")
    ap.add_argument("--no-mx-prepared", action="store_true",
                    help="skip the legs on MXFP8 fragment panels")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs one GPU's share of the layer; "
                          "--gpus above 1 is not supported (multi-GPU sharding is a design only)"}))
        sys.exit(2)

    import torch
    import moe_inputs as mi
    from prefill_sigmoid_router_amd import binding as B

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    B.load_library()

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    head = mi.CONFIGS[args.workload]
    print(f"bench: generating weights E={head.E} H={head.H} I={head.I}", file=sys.stderr, flush=True)
    full = mi.make_layer(head, device=dev, seed=0)
    weights = {"w13": full["w13"], "w2": full["w2"], "router_w": full["router_w"],
               "norm_w": full["norm_w"]}
    del full
    torch.cuda.synchronize()

    # read probes over the resident W13 (the bytes the up GEMM streams), once before the
    # legs and once after them (a box that has run for minutes can read at another rate);
    # each probe keeps the better of its two passes
    print("bench: timing the HBM read probes", file=sys.stderr, flush=True)
    probes = read_probes(torch, dev, weights["w13"])

    print(f"bench: timing {args.workload}", file=sys.stderr, flush=True)
    res = run_workload(B, mi, torch, head, weights, args.steps, args.warmup, dev)
    sweep = {}
    if not args.no_sweep:
        for name in SWEEP:
            if name == args.workload:
                continue
            print(f"bench: timing {name}", file=sys.stderr, flush=True)
            sweep[name] = run_workload(B, mi, torch, mi.CONFIGS[name], weights,
                                       max(3, args.steps // 2), max(1, args.warmup // 2), dev)

    # (leg dict, workload, result, up kernel, weight format) of the fragment-panel legs, whose
    # roofline objects are filled in once the read probes have run
    leg_roofs = []
    mx_line = None
    if not args.no_mx:
        # the same layer with MXFP8 expert weights (quantized on the device)
        print("bench: quantizing the experts to MXFP8 and timing decode_m8", file=sys.stderr,
              flush=True)
        mx = []
        for name in ("w13", "w2"):
            w = weights[name]
            c = torch.empty(tuple(w.shape), dtype=torch.uint8, device=dev)
            sc = torch.empty(tuple(w.shape[:-1]) + (w.shape[-1] // 32,), dtype=torch.uint8,
                             device=dev)
            B.moe_mx_quantize(w, c, sc)
            mx += [c, sc]
        torch.cuda.synchronize()
        dcfg = mi.CONFIGS["decode_m8"]
        r = run_workload(B, mi, torch, dcfg, weights, args.steps, args.warmup, dev, mx=mx)
        mx_line = _rounded(r)
        mx_line["weights"] = "MXFP8 (E4M3 + E8M0 per 32 values along K), activations bf16"
        mx_line["up_kernel"] = up_kernel_name(B, dcfg, mx=True)
        mx_line["up_hbm_frac"] = round(r["up_gbs"] / HBM_PEAK_GBS, 4)
        if not args.no_sweep:
            mx_sweep = {}
            for name in SWEEP:
                print(f"bench: timing {name} with MXFP8 experts", file=sys.stderr, flush=True)
                c = mi.CONFIGS[name]
                rs = run_workload(B, mi, torch, c, weights, max(3, args.steps // 2),
                                  max(1, args.warmup // 2), dev, mx=mx)
                mx_sweep[name] = _rounded(rs)
                mx_sweep[name]["tile_rows"] = B.moe_gemm_tile_rows_mx(c.M, c.E, c.top_k, c.I)
                mx_sweep[name]["up_kernel"] = up_kernel_name(B, c, mx=True)
                mx_sweep[name]["up_hbm_frac"] = round(rs["up_gbs"] / HBM_PEAK_GBS, 4)
            mx_line["sweep"] = mx_sweep
        if not args.no_mx_prepared:
            # the same MXFP8 codes re-laid-out once into fragment panels
            print("bench: re-laying-out the MXFP8 experts into panels", file=sys.stderr,
                  flush=True)
            E, H, I = head.E, head.H, head.I
            mxp = [torch.empty(n, dtype=torch.uint8, device=dev)
                   for n in B.moe_mx_prepared_bytes(E, H, I)]
            B.moe_mx_prepare_weights(*mx, E, H, I, *mxp)
            torch.cuda.synchronize()
            del mx
            torch.cuda.empty_cache()
            mxp_line = {}
            for name in (head.name,) + (() if args.no_sweep else SWEEP):
                if name in mxp_line:
                    continue
                print(f"bench: timing {name} on MXFP8 panels", file=sys.stderr, flush=True)
                c = mi.CONFIGS[name]
                quick = name != head.name
                r = run_workload(B, mi, torch, c, weights,
                                 max(3, args.steps // 2) if quick else args.steps,
                                 max(1, args.warmup // 2) if quick else args.warmup, dev,
                                 mxp=mxp)
                mxp_line[name] = _rounded(r)
                mxp_line[name]["up_hbm_frac"] = round(r["up_gbs"] / HBM_PEAK_GBS, 4)
                mxp_line[name]["up_mfma_frac"] = round(r["up_tflops"] / BF16_PEAK_TFLOPS, 4)
                mxp_line[name]["down_hbm_frac"] = round(r["down_gbs"] / HBM_PEAK_GBS, 4)
                mxp_line[name]["up_kernel"] = (
                    f"expert_frag_kernel<{B.moe_gemm_tile_rows_panels(c.M, c.E, c.top_k, c.I, 8)}, "
                    "true, ..., MXFP8>")
                leg_roofs.append((mxp_line, name, r, mxp_line[name]["up_kernel"], "mx8"))
            mxp_line["weights"] = ("MXFP8 (E4M3 + E8M0 per 32 values along K, fragment "
                                   "panels), activations bf16")
            mx_line["prepared_panels"] = mxp_line
            del mxp
        else:
            del mx
        torch.cuda.empty_cache()

    prep_line = None
    if not args.no_prepared:
        # the same layer on weights re-laid-out once into fragment panels (moe_forward_prepared)
        print("bench: preparing fragment-panel weights", file=sys.stderr, flush=True)
        E, H, I = head.E, head.H, head.I
        p13 = torch.empty(B.moe_prepared_w13_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
        p2 = torch.empty(B.moe_prepared_w2_bytes(E, H, I) // 2, dtype=torch.bfloat16, device=dev)
        B.moe_prepare_weights(weights["w13"], weights["w2"], p13, p2)
        torch.cuda.synchronize()
        prep_line = {}
        for name in (head.name,) + (() if args.no_sweep else SWEEP):
            if name in prep_line:
                continue
            print(f"bench: timing {name} on prepared weights", file=sys.stderr, flush=True)
            c = mi.CONFIGS[name]
            quick = name != head.name
            r = run_workload(B, mi, torch, c, weights,
                             max(3, args.steps // 2) if quick else args.steps,
                             max(1, args.warmup // 2) if quick else args.warmup, dev,
                             prepared=(p13, p2))
            prep_line[name] = _rounded(r)
            prep_line[name]["up_hbm_frac"] = round(r["up_gbs"] / HBM_PEAK_GBS, 4)
            prep_line[name]["up_mfma_frac"] = round(r["up_tflops"] / BF16_PEAK_TFLOPS, 4)
            prep_line[name]["down_hbm_frac"] = round(r["down_gbs"] / HBM_PEAK_GBS, 4)
            prep_line[name]["up_kernel"] = (
                f"expert_frag_kernel<{B.moe_gemm_tile_rows_panels(c.M, c.E, c.top_k, c.I, 16)}, "
                "true, ...>")
            leg_roofs.append((prep_line, name, r, prep_line[name]["up_kernel"], "bf16"))
        del p13, p2
        torch.cuda.empty_cache()

    mx4_line = None
    if not args.no_mx4:
        # the same layer with MXFP4 expert weights (quantized on the device into panels)
        print("bench: quantizing the experts to MXFP4", file=sys.stderr, flush=True)
        E, H, I = head.E, head.H, head.I
        q = [torch.empty(n, dtype=torch.uint8, device=dev) for n in B.moe_mx4_weight_bytes(E, H, I)]
        B.moe_mx4_quantize(weights["w13"], weights["w2"], *q)
        torch.cuda.synchronize()
        mx4_line = {}
        for name in (head.name,) + (() if args.no_sweep else SWEEP):
            if name in mx4_line:
                continue
            print(f"bench: timing {name} with MXFP4 experts", file=sys.stderr, flush=True)
            c = mi.CONFIGS[name]
            quick = name != head.name
            r = run_workload(B, mi, torch, c, weights,
                             max(3, args.steps // 2) if quick else args.steps,
                             max(1, args.warmup // 2) if quick else args.warmup, dev, mx4=q)
            mx4_line[name] = _rounded(r)
            mx4_line[name]["up_hbm_frac"] = round(r["up_gbs"] / HBM_PEAK_GBS, 4)
            mx4_line[name]["down_hbm_frac"] = round(r["down_gbs"] / HBM_PEAK_GBS, 4)
            mx4_line[name]["up_kernel"] = (
                f"expert_frag_kernel<{B.moe_gemm_tile_rows_panels(c.M, c.E, c.top_k, c.I, 4)}, "
                "true, ..., MXFP4>")
            leg_roofs.append((mx4_line, name, r, mx4_line[name]["up_kernel"], "mx4"))
        mx4_line["weights"] = ("MXFP4 (E2M1 + E8M0 per 32 values along K, fragment panels), "
                               "activations bf16")
        del q
        torch.cuda.empty_cache()

    print("bench: timing the HBM read probes again", file=sys.stderr, flush=True)
    probes = {k: max(v, probes[k]) for k, v in read_probes(torch, dev, weights["w13"]).items()}
    read_gbs = max(probes.values())

    head_kernel = up_kernel_name(B, head)
    roof = roofline(res, head_kernel, read_gbs,
                    load_profile(f"traffic_expert_up_{head.name}.json", head.name, head_kernel))
    roof["read_probes_gbs"] = {k: round(g, 1) for k, g in probes.items()}
    for line_d, name, r, kernel, fmt in leg_roofs:
        line_d[name]["roofline"] = roofline(
            r, kernel, read_gbs,
            load_profile(f"traffic_expert_frag_up_{fmt}_{name}.json", name, kernel))
    sweep_out = {}
    for name, r in sweep.items():
        c = mi.CONFIGS[name]
        sweep_out[name] = _rounded(r)
        kernel = up_kernel_name(B, c)
        sweep_out[name]["roofline"] = roofline(
            r, kernel, read_gbs, load_profile(f"traffic_expert_up_{name}.json", name, kernel))

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(mi, torch, weights, dev, sweep=not args.no_sweep)

    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "us_per_layer": round(res["us_per_layer"], 2),
        "layer_us_p10_p50_p90": res["layer_us_p10_p50_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, random init)",
        "config": {"workload": head.name, "M": head.M, "H": head.H, "E": head.E,
                   "top_k": head.top_k, "I": head.I, "block": head.block,
                   "routing": "uniform" if head.zipf_s is None else f"zipf({head.zipf_s})",
                   "touched_experts": res["touched_experts"], "plan_rows": res["plan_rows"],
                   "parallelism": "single GPU"},
        "stages_us": res["stages_us"],
        "align": res["align"],
        "layer_hbm_frac": round(res["layer_hbm_frac"], 4),
        "layer_gbs": round(res["layer_gbs"], 1),
        "layer_frac_of_measured_read": round(res["layer_gbs"] / read_gbs, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "sweep": sweep_out,
        "mxfp8_decode": mx_line,
        "prepared_weights": prep_line,
        "mxfp4": mx4_line,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
