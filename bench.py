"""Benchmark of one routed-MoE layer (router -> align -> up+SwiGLU -> down -> finalize) on
one MI355X, through the C ABI.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload decode_m8]
                    [--no-sweep] [--no-cpu-baseline] [--no-mx]

Prints ONE JSON line.  A step is one moe_forward call (all five kernels) over resident
inputs of the workload; K steps are timed between two synchronisations (wall clock and
HIP events on the launch stream, the larger is used).  A second pass of K steps records
six HIP events per step around the five kernels for the per-kernel durations (an event
between two kernels adds a few microseconds of idle, so that pass is not the headline).  `value` is tokens/s
of the headline workload (decode, M=8); `sweep` holds the same measurement at M=128,
512 and 2048 on the same weights.  `roofline` is for the dominant kernel (the grouped
up-GEMM + SwiGLU, which streams W13) against the 8 TB/s HBM peak, and against the read
rate this device reaches with a plain streaming read of the resident W13
(`measured_read_peak`, from the probe library built next to the layer's);
`cpu_baseline` is the CPU oracle timed on a bounded sample of the decode workload.  `mxfp8_decode` times the same decode layer with
the expert weights quantized to MXFP8 (moe_forward_mx); it is a separate measurement, not
the headline, whose weights are bf16.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "MoE-layer tokens/s and µs/layer at M=8/128/2048; % HBM or MFMA roofline"
STAGES = ("route", "align", "up", "down", "finalize")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_expert_up_decode_m8.json")


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def weight_bytes_per_value(mx):
    """bf16: 2 bytes; MXFP8: one E4M3 byte plus one scale byte per 32 values."""
    return 1 + 1 / 32 if mx else 2


def layer_bytes(cfg, M, touched, mx=False):
    """Algorithmic HBM bytes of one layer: touched experts' W13+W2, the router weight,
    x, residual and out rows, and the norm weight."""
    per_expert = 3 * cfg.I * cfg.H * weight_bytes_per_value(mx)
    return int(touched * per_expert) + cfg.E * cfg.H * 2 + 3 * M * cfg.H * 2 + cfg.H * 2


def up_bytes(cfg, M, touched, mx=False):
    """Algorithmic bytes of the up kernel: W13 of every touched expert, each token's x
    row once, and one bf16 act row per (token, pick)."""
    return (int(touched * 2 * cfg.I * cfg.H * weight_bytes_per_value(mx)) + M * cfg.H * 2
            + M * cfg.top_k * cfg.I * 2)


def layer_flops(cfg, M):
    return 2 * M * cfg.E * cfg.H + 6 * M * cfg.top_k * cfg.H * cfg.I


def run_workload(B, mi, torch, cfg, weights, steps, warmup, dev, mx=None):
    """Times moe_forward (bf16 experts), or moe_forward_mx when `mx` holds the MXFP8
    (w13 codes, w13 scales, w2 codes, w2 scales)."""
    L = mi.make_layer(cfg, device=dev, seed=0, with_experts=False)
    L.update(weights)
    M, H, E, I, k, blk = cfg.M, cfg.H, cfg.E, cfg.I, cfg.top_k, cfg.block
    cap = B.moe_align_capacity(M, k, E, blk)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    ws = torch.empty(B.moe_workspace_bytes(M, H, E, I, k, blk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(events=None):
        if mx is None:
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
    ms = max(wall_ms, span_ms)
    touched = int(torch.unique(ids).numel())
    counts = torch.bincount(ids.flatten().long(), minlength=E)
    lb = layer_bytes(cfg, M, touched, mx is not None)
    ub = up_bytes(cfg, M, touched, mx is not None)
    return {
        "M": M, "ms_per_step": ms, "us_per_layer": ms * 1e3, "tokens_per_s": M / (ms / 1e3),
        "wall_ms": wall_ms, "event_span_ms": span_ms,
        "stages_us": {n: round(v * 1e3, 2) for n, v in stage_ms.items()},
        "touched_experts": touched, "max_expert_count": int(counts.max().item()),
        "plan_rows": int(sum(((c + blk - 1) // blk) * blk for c in counts.tolist())),
        "layer_bytes": lb, "layer_gbs": lb / (ms / 1e3) / 1e9,
        "layer_hbm_frac": lb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac": layer_flops(cfg, M) / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        "up_bytes": ub, "up_us": stage_ms["up"] * 1e3,
        "up_gbs": ub / (stage_ms["up"] / 1e3) / 1e9,
    }


def cpu_baseline(mi, torch):
    """The oracle (plan-based forward, fp64 numpy) on the host over the decode batch."""
    from oracle import moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cfg = mi.CONFIGS["decode_m8"]
    L = mi.make_layer(cfg, device="cpu", seed=0, with_experts=False)
    bits = mi.bf16_bits
    xb, rb = bits(L["x"]), bits(L["residual"])
    wrb, gb = bits(L["router_w"]), bits(L["norm_w"])
    ids, _, _ = orc.route(xb, wrb, None, cfg.top_k)
    need = sorted(set(int(e) for e in ids.ravel()))
    w13 = {e: bits(mi.expert_w13(cfg, e, "cpu", 0)) for e in need}   # generated before timing
    w2 = {e: bits(mi.expert_w2(cfg, e, "cpu", 0)) for e in need}
    times = []
    while len(times) < 3 and sum(times) < 20.0:
        t0 = time.perf_counter()
        orc.forward(xb, wrb, None, w13, w2, rb, gb, cfg.eps, cfg.top_k, cfg.block)
        times.append(time.perf_counter() - t0)
    sec = sorted(times)[len(times) // 2]
    return {
        "value": cfg.M / sec, "unit": "tokens/s", "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"decode_m8 workload (host-generated, same recipe): all {cfg.M} tokens through "
                   f"the whole layer, {len(need)} experts, fp64 numpy with bf16 weights decoded "
                   f"inside the timed region; median of {len(times)} runs = {sec:.2f} s; "
                   f"BLAS threads {blas_threads}, host cpus {len(os.sched_getaffinity(0))}"),
    }


def read_probe_gbs(torch, dev, gib=4, reps=5, buf=None):
    """Achievable HBM read rate on this device: best of `reps` timed passes of the read
    probe (prefill_sigmoid_router_amd/probe/read_bw.hip) over `buf` (a resident tensor,
    read as raw bytes) or, without one, a fresh `gib` GiB buffer."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "prefill_sigmoid_router_amd", "libmoe_probe.so"))
    lib.moe_probe_read.restype = ctypes.c_int
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.moe_probe_read_grid.restype = ctypes.c_int
    own = buf is None
    if own:
        buf = torch.ones((gib << 30) // 4, dtype=torch.int32, device=dev)
    n = buf.numel() * buf.element_size() // 16 * 16
    sink = torch.empty(lib.moe_probe_read_grid(), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def once():
        st = lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()), n,
                                ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"moe_probe_read failed with status {st}")

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
    del sink
    if own:
        del buf
    return n / (best * 1e-3) / 1e9


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, "prefill_sigmoid_router_amd", "csrc", t.get("source_file", ""))
    if not os.path.isfile(src) or t.get("source_sha256_16") != source_hash(src):
        return None     # the kernel changed since the counters were taken
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_m8")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the decode leg with MXFP8 expert weights")
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

    print(f"bench: timing {args.workload}", file=sys.stderr, flush=True)
    res = run_workload(B, mi, torch, head, weights, args.steps, args.warmup, dev)
    sweep = {}
    if not args.no_sweep:
        for name in ("batch_m128", "batch_m512", "prefill_m2048"):
            if name == args.workload:
                continue
            print(f"bench: timing {name}", file=sys.stderr, flush=True)
            r = run_workload(B, mi, torch, mi.CONFIGS[name], weights, max(3, args.steps // 2),
                             max(1, args.warmup // 2), dev)
            sweep[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}

    mx_line = None
    if not args.no_mx:
        # the same decode layer with MXFP8 expert weights (quantized on the device)
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
        r = run_workload(B, mi, torch, mi.CONFIGS["decode_m8"], weights, args.steps, args.warmup,
                         dev, mx=mx)
        mx_line = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        mx_line["weights"] = "MXFP8 (E4M3 + E8M0 per 32 values along K), activations bf16"
        mx_line["up_kernel"] = "expert_mx_decode_kernel<true> (codes copied into LDS, 32-row tiles)"
        mx_line["up_hbm_frac"] = round(r["up_gbs"] / HBM_PEAK_GBS, 4)
        if not args.no_sweep:
            mx_sweep = {}
            for name in ("batch_m128", "batch_m512", "prefill_m2048"):
                print(f"bench: timing {name} with MXFP8 experts", file=sys.stderr, flush=True)
                rs = run_workload(B, mi, torch, mi.CONFIGS[name], weights, max(3, args.steps // 2),
                                  max(1, args.warmup // 2), dev, mx=mx)
                mx_sweep[name] = {k: (round(v, 4) if isinstance(v, float) else v)
                                  for k, v in rs.items()}
                mx_sweep[name]["tile_rows"] = B.moe_gemm_tile_rows_mx(
                    rs["M"], head.E, head.top_k, head.I)
            mx_line["sweep"] = mx_sweep
        del mx
        torch.cuda.empty_cache()

    # the read probe over the resident W13 (the bytes the up GEMM streams)
    print("bench: timing the HBM read probe", file=sys.stderr, flush=True)
    read_gbs = read_probe_gbs(torch, dev, buf=weights["w13"])
    traffic = load_traffic()
    rows = B.moe_gemm_tile_rows(head.M, head.E, head.top_k, head.I)
    if B.moe_forward_self_routes(head.M, head.E, head.top_k, head.I):
        up_kernel = f"expert_up_selfroute_kernel<{rows}, ...>, align fused in,"
    elif rows == 16:
        up_kernel = "expert_up_stream_kernel"
    else:
        up_kernel = f"expert_tiled_kernel<{rows}, ..., true, ...>"
    if traffic is not None and traffic.get("workload") != head.name:
        traffic = None  # counters were taken on another workload
    roof = {
        "bound": "hbm", "kernel": f"{up_kernel} (grouped up-GEMM + SwiGLU)",
        "achieved": round(res["up_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(res["up_gbs"] / HBM_PEAK_GBS, 4),
        "traffic": None if traffic is None else traffic.get("traffic_gbs"),
        "traffic_bytes_per_launch": None if traffic is None else traffic.get("traffic_bytes_per_launch"),
        "algorithmic_bytes_per_launch": res["up_bytes"], "avg_launch_us": round(res["up_us"], 2),
        "measured_read_peak": round(read_gbs, 1),
        "frac_of_measured_read": round(res["up_gbs"] / read_gbs, 4),
    }
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(mi, torch)

    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "us_per_layer": round(res["us_per_layer"], 2),
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
        "layer_hbm_frac": round(res["layer_hbm_frac"], 4),
        "layer_gbs": round(res["layer_gbs"], 1),
        "layer_frac_of_measured_read": round(res["layer_gbs"] / read_gbs, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "mxfp8_decode": mx_line,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
