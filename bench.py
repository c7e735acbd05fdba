"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload v3] [--cpu-sample S]

One step = one whole layer forward (route -> dispatch -> routed expert FFN ->
shared expert -> combine) over one batch of T tokens, inputs and weights
resident in HBM.  Prints one JSON line: tokens/s for the whole step, per-stage
times from HIP events on the stream the kernels run on, the roofline of the
dominant kernel (the routed up-projection GEMM + SwiGLU), and the CPU oracle
timed on a bounded sample of the same workload.
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

METRIC = "MoE-layer fwd tokens/sec on 1 MI355X; GEMM MFMA % peak; route/permute GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
HASH_SEED = 7

# HBM traffic of the routed up-projection launch, per launch, from two
# rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over
#   python3 bench.py [--workload W] --steps 2 --warmup 1 --cpu-sample 0 --copy-probe
# Each counter is scaled by what it reads for the copy probe (a plain 2 GiB
# elementwise copy run in the same process): on gfx950 FETCH_SIZE reports half
# of the bytes a full-line read moves, WRITE_SIZE reports them exactly.  A
# record holds only for the kernel sources it was taken from: any change to them
# turns the reported traffic into null until the passes are taken again.
_SHARED_SOURCES = ("moe_expert_routing_sqrt_amd/csrc/gemm_common.h",
                   "moe_expert_routing_sqrt_amd/csrc/common.h",
                   "moe_expert_routing_sqrt_amd/build.py")
TRAFFIC = {
    "v3": {"sources": ("moe_expert_routing_sqrt_amd/csrc/ffn_bf16.hip",) + _SHARED_SOURCES,
           "sources_sha256": "23cf24a5e55cfb4ef500be7805ed0550240ecd14a608aa5a728a97b5c461a077",
           "fetch_kib": 18642588.6, "fetch_scale": 1.99997,
           "write_kib": 524627.8, "write_scale": 1.0},
    "v3_fp8": {"sources": ("moe_expert_routing_sqrt_amd/csrc/gemm_fp8p.hip",) + _SHARED_SOURCES,
               "sources_sha256": "d66ee96f45d1a738a35ef06a243694d553fee477e2f3d1d052995c4258c0b504",
               "fetch_kib": 10636418.9, "fetch_scale": 1.99997,
               "write_kib": 274533.6, "write_scale": 1.0},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3")
    ap.add_argument("--cpu-sample", type=int, default=512, help="tokens the CPU oracle runs (0: skip)")
    ap.add_argument("--router", default="topk", choices=("topk", "hash"),
                    help="topk: the affinity router; hash: experts from a hash of synthetic token ids")
    ap.add_argument("--backward", action="store_true",
                    help="also time forward+backward steps (bf16 top-k workload) and report the backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 2 GiB copy (counter calibration for --pmc passes)")
    ap.add_argument("--up-variants", action="store_true",
                    help="instead of the bench: time the routed up-projection against the same rows in "
                         "equal shares per expert and against one expert's weights (one JSON line)")
    return ap.parse_args()


def workload_name(cfg, router="topk") -> str:
    s = (f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} G={cfg.G} k={cfg.k} M={cfg.M} d_ff={cfg.d_ff} "
         f"{cfg.dtype}")
    if router == "hash":
        s += ", hash router (Philox of Zipf(1.1) token ids over 65536)"
    if cfg.local:
        s += f" experts [{cfg.e_begin},{cfg.e_end}) only"
    else:
        s += f" + {cfg.n_shared} shared expert"
    if cfg.skew:
        s += ", Zipf(1.2) logit offset"
    return s


def algorithmic(cfg):
    """Per-launch algorithmic work of each stage: the bytes the method must move
    or the FLOPs it must compute, padding and re-reads excluded."""
    T, d, E, k, d_ff = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    P = T * k if not cfg.local else None
    act = 4 if cfg.dtype == "f32" else 2
    # packed-row bytes: e4m3 codes plus one fp32 scale per 128 columns for fp8
    packed = d + 4 * (d // 128) if cfg.dtype == "fp8" else d * act
    wbytes = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.dtype]
    return {
        "route_flops": 2 * T * d * E,
        "route_select_bytes": T * E * 4 + E * 4 + T * k * 8 + ((T + 63) // 64) * E * 4,
        "dispatch_bytes": lambda rows: T * d * act + rows * packed + 12 * T * k,
        "ffn_up_flops": lambda rows: 4 * d * d_ff * rows,
        # packed rows in, the local experts' W1/W3 once, h out (+ scales for fp8)
        "ffn_up_bytes": lambda rows: rows * packed + (cfg.e_end - cfg.e_begin) * 2 * d_ff * d * wbytes
        + rows * (d_ff + 4 * (d_ff // 128) if cfg.dtype == "fp8" else d_ff * act)
        + ((cfg.e_end - cfg.e_begin) * 2 * d_ff * d // (128 * 128) * 4 if cfg.dtype == "fp8" else 0),
        "ffn_down_flops": lambda rows: 2 * d * d_ff * rows,
        "shared_flops": 6 * d * d_ff * T,
        "combine_bytes": lambda rows: rows * d * act + 8 * T * k + (T * d * act if not cfg.local else 0)
        + T * d * (4 * 2 if cfg.local else act),
        "pairs": P,
    }


def sources_digest(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return ""
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic(cfg, up_bytes):
    """Counter-measured HBM bytes per routed up-projection launch, or None."""
    rec = TRAFFIC.get(cfg.name)
    if rec is None or rec["sources_sha256"] != sources_digest(rec["sources"]):
        return None
    fetch = rec["fetch_kib"] * 1024 * rec["fetch_scale"]
    write = rec["write_kib"] * 1024 * rec["write_scale"]
    return {"bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "vs_algorithmic_bytes": (fetch + write) / up_bytes}


def copy_probe(torch, dev):
    """A plain elementwise copy of known size: 2 GiB read, 2 GiB written per launch."""
    n = (2 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print("copy probe: 3 launches of a 2 GiB fp32 negation", file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()


def backward_bench(a, cfg, layer, x, ev, torch, alg, rows):
    """Forward + backward steps of the bf16 top-k layer; the backward's stages
    timed with events (combine, routed experts, shared expert, dispatch + gate)."""
    g = torch.randn((cfg.T, cfg.d), device=x.device, dtype=torch.float32).to(torch.bfloat16)
    for _ in range(max(1, a.warmup)):
        layer.forward(x, save_for_backward=True)
        layer.backward(x, g)
    torch.cuda.synchronize()
    steps = max(5, a.steps // 5)
    fm = [[ev() for _ in range(7)] for _ in range(steps)]
    bm = [[ev() for _ in range(5)] for _ in range(steps)]
    s0, s1 = ev(), ev()
    s0.record()
    for i in range(steps):
        layer.forward(x, marks=fm[i], save_for_backward=True)
        layer.backward(x, g, marks=bm[i])
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    names = ("combine_bwd", "routed_experts_bwd", "shared_expert_bwd", "dispatch_gate_bwd")
    st = {n: sum(m[i].elapsed_time(m[i + 1]) for m in bm) / steps for i, n in enumerate(names)}
    bwd_ms = sum(st.values())
    # expert backward products (the forward kept [a | u]): d_h (2 d d_ff per
    # row), d_x (4), dW2 (2), dW13 (4) = 12 d d_ff per row
    fl = 12 * cfg.d * cfg.d_ff
    peak = PEAK_BF16_TFLOPS
    tf = lambda flops, t: flops / (t * 1e-3) / 1e12
    return {"steps": steps, "fwd_bwd_ms_per_step": ms, "fwd_bwd_tokens_per_s": cfg.T / (ms * 1e-3),
            "bwd_ms": bwd_ms, "stages_ms": st,
            "routed_experts_tflops": tf(fl * rows, st["routed_experts_bwd"]),
            "routed_experts_frac_mfma": tf(fl * rows, st["routed_experts_bwd"]) / peak,
            "shared_expert_tflops": tf(fl * cfg.T, st["shared_expert_bwd"]),
            "train_forward_ms": sum(m[0].elapsed_time(m[6]) for m in fm) / steps,
            "flops_note": "12*d*d_ff per row: d_h + d_x + dW2 + dW13 (the training forward keeps [a|u])"}


def cpu_baseline(cfg, inp, ex, S, ids=None):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import combine as OC, dispatch as OD, ffn as OF, hash_route as OH, route as OR

    S = min(S, cfg.T)
    x = inp["x"][:S].float().cpu().numpy()
    wg = inp["w_gate"].cpu().numpy()
    bias = inp["bias"].cpu().numpy()
    off = None if inp["logit_offset"] is None else inp["logit_offset"].cpu().numpy()
    # weights as the GPU holds them, copied to host memory before timing; the
    # oracle converts each expert to fp64 as it streams through them
    w13_h = ex["w13"].cpu()
    w2_h = ex["w2"].cpu()
    sh13 = ex["sh_w13"][0].cpu()
    sh2 = ex["sh_w2"][0].cpu()
    f = lambda t: t.float().numpy()
    st = {}

    def route_dispatch():
        if ids is None:
            _, idx_, w_ = OR.route(x, wg, bias, cfg.G, cfg.M, cfg.k, cfg.gk, off)
        else:
            idx_, w_ = OH.hash_route(ids[:S], cfg.E, cfg.k, HASH_SEED)
        ta = time.perf_counter()
        disp = OD.dispatch(idx_, cfg.E, cfg.e_begin, cfg.e_end)
        return idx_, w_, disp, ta

    t0 = time.perf_counter()
    idx, w, (counts, offsets, dest, src), t1 = route_dispatch()
    xp = OD.pack(x, src)
    t2 = time.perf_counter()
    yp, _ = OF.grouped_ffn(xp, offsets, None, None, weight_fn=lambda i: (f(w13_h[i]), f(w2_h[i])))
    t3 = time.perf_counter()
    ysh = None
    if not cfg.local:
        ysh, _ = OF.expert_forward(x, f(sh13), f(sh2))
    t4 = time.perf_counter()
    if cfg.local:
        out = OC.combine(yp, dest, w, out_init=np.zeros((S, cfg.d)))
    else:
        out = OC.combine(yp, dest, w, ysh=ysh)
    t5 = time.perf_counter()
    t = t5 - t0
    for name, a, b in (("route", t0, t1), ("dispatch", t1, t2), ("routed_experts", t2, t3),
                       ("shared_expert", t3, t4), ("combine", t4, t5)):
        st[name] = {"seconds": b - a, "tokens_per_s": S / max(b - a, 1e-9)}
    # route and dispatch again on one core
    with threadpool_limits(1):
        u0 = time.perf_counter()
        _, _, (_, _, _, src1), u1 = route_dispatch()
        OD.pack(x, src1)
        u2 = time.perf_counter()
    st["route_one_core"] = {"seconds": u1 - u0, "tokens_per_s": S / max(u1 - u0, 1e-9)}
    st["dispatch_one_core"] = {"seconds": u2 - u1, "tokens_per_s": S / max(u2 - u1, 1e-9)}
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of the {cfg.T} tokens, whole layer (route, dispatch, all routed "
                      f"experts they reach, shared expert, combine) in fp64 numpy; {t:.1f} s; "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus",
            "seconds": t, "stages": st}


def up_variants(torch, M, cfg, layer, x, ids):
    """The routed up-projection of one forward, then the same packed rows split
    equally over the experts (every tile full, every expert's own weights) and
    given to one expert (one weight set), in that order: the mean of five
    back-to-back launches each, printed as one JSON line.  Three forwards
    first bring the clocks up."""
    for _ in range(3):
        layer.forward(x, token_ids=ids)
    torch.cuda.synchronize()
    b = layer.dbufs
    rows = int(b["offsets"][-1].item())
    n = layer.w13.shape[0]
    dev = x.device
    first = lambda t: None if t is None else t[:1]
    variants = [("routed", b["offsets"], layer.w13, layer.w13_s)]
    if rows % n == 0:
        variants.append(("uniform", torch.arange(0, rows + 1, rows // n, dtype=torch.int32, device=dev),
                         layer.w13, layer.w13_s))
    variants.append(("dense", torch.tensor([0, rows], dtype=torch.int32, device=dev), layer.w13[:1],
                     first(layer.w13_s)))
    flops = 4 * cfg.d * cfg.d_ff * rows
    res = {}
    for name, off, w13, w13_s in variants:
        # five back-to-back launches between two events on the launch stream
        # (no host gap between them); the first (untimed) brings the clocks up
        run = lambda: M.expert_ffn(off, layer.max_rows, b["xp"], w13, layer.w2, layer.dtype,
                                   xp_scale=b["xp_scale"], w13_scale=w13_s, w2_scale=layer.w2_s, h=layer.h,
                                   h_scale=layer.h_s, yp=layer.yp, stages=M.MOE_FFN_UP)
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res[name] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}
    print(json.dumps({"up_variants": res, "workload": workload_name(cfg), "rows": rows}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    import moe_expert_routing_sqrt_amd as M
    from moe_inputs import configs as C, generate as gen

    cfg = C.get(a.workload)
    dev = torch.device("cuda:0")
    if a.copy_probe:
        copy_probe(torch, dev)
    t_setup = time.perf_counter()
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                       inp["bias"], ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"],
                       logit_offset=inp["logit_offset"], e_begin=cfg.e_begin, e_end=cfg.e_end,
                       group_topk=cfg.gk, router=a.router, hash_seed=HASH_SEED)
    x = inp["x"]
    ids = gen.token_ids(cfg, device=dev) if a.router == "hash" else None
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f}s: {workload_name(cfg, a.router)}", file=sys.stderr, flush=True)
    if a.up_variants:
        up_variants(torch, M, cfg, layer, x, ids)
        return

    for _ in range(a.warmup):
        layer.forward(x, token_ids=ids)
    torch.cuda.synchronize()
    print(f"warmup {a.warmup} done", file=sys.stderr, flush=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [[ev() for _ in range(7)] for _ in range(a.steps)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(a.steps):
        layer.forward(x, marks=marks[i], token_ids=ids)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / a.steps
    per_step = sorted(m[0].elapsed_time(m[6]) for m in marks)
    median_ms = per_step[len(per_step) // 2]
    print(f"timed {a.steps} steps: {ms_per_step:.3f} ms/step (host wall {wall / a.steps * 1e3:.3f})",
          file=sys.stderr, flush=True)

    # the balancing step that follows a forward (moe_bias_update on the route's
    # block counts); gamma = 0 keeps the workload fixed across repetitions
    bu0, bu1 = ev(), ev()
    reps = 50
    load_buf = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    bu0.record()
    for _ in range(reps):
        M.bias_update(layer.block_counts, layer.bias, 0.0, load_buf)
    bu1.record()
    torch.cuda.synchronize()
    bu_us = bu0.elapsed_time(bu1) / reps * 1e3
    nblk = layer.block_counts.shape[0]
    bu_bytes = nblk * cfg.E * 4 + cfg.E * 4 * 3

    names = ("route", "dispatch", "ffn_up", "ffn_down", "shared", "combine")
    st_ms = {n: sum(m[i].elapsed_time(m[i + 1]) for m in marks) / a.steps for i, n in enumerate(names)}
    rows = int(layer.dbufs["offsets"][-1].item())
    alg = algorithmic(cfg)
    peak_mm = PEAK_FP8_TFLOPS if cfg.dtype == "fp8" else PEAK_BF16_TFLOPS
    tf = lambda flops, ms: flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    gbs = lambda byts, ms: byts / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    stages = {
        "route": ({"ms": st_ms["route"], "gate_tflops": tf(alg["route_flops"], st_ms["route"])}
                  if a.router == "topk" else
                  {"ms": st_ms["route"], "kind": "hash router",
                   "bytes": cfg.T * 4 + cfg.T * cfg.k * 8 + ((cfg.T + 63) // 64) * cfg.E * 4}),
        "dispatch": {"ms": st_ms["dispatch"], "gb_s": gbs(alg["dispatch_bytes"](rows), st_ms["dispatch"])},
        "ffn_up": {"ms": st_ms["ffn_up"], "tflops": tf(alg["ffn_up_flops"](rows), st_ms["ffn_up"])},
        "ffn_down": {"ms": st_ms["ffn_down"], "tflops": tf(alg["ffn_down_flops"](rows), st_ms["ffn_down"])},
        "shared": {"ms": st_ms["shared"], "tflops": tf(alg["shared_flops"] if layer.has_shared else 0,
                                                        st_ms["shared"])},
        "combine": {"ms": st_ms["combine"], "gb_s": gbs(alg["combine_bytes"](rows), st_ms["combine"])},
    }
    for s in ("dispatch", "combine"):
        stages[s]["frac_hbm"] = stages[s]["gb_s"] / PEAK_HBM_GBS
    for s in ("ffn_up", "ffn_down", "shared"):
        stages[s]["frac_mfma"] = stages[s]["tflops"] / peak_mm
    gemm_ms = st_ms["ffn_up"] + st_ms["ffn_down"] + st_ms["shared"]
    gemm_flops = alg["ffn_up_flops"](rows) + alg["ffn_down_flops"](rows) + (alg["shared_flops"] if layer.has_shared else 0)
    up = stages["ffn_up"]
    up_traffic = traffic(cfg, alg["ffn_up_bytes"](rows))
    result = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": median_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "e4m3"}[cfg.dtype],
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02^2) weights, U(-0.1,0.1) bias)",
        "config": {"workload": workload_name(cfg, a.router), "router": a.router, "T": cfg.T, "d": cfg.d, "E": cfg.E, "G": cfg.G,
                   "k": cfg.k, "M": cfg.M, "d_ff": cfg.d_ff, "routed_rows": rows},
        "roofline": {"kernel": "routed up-projection GEMM + SwiGLU (moe_expert_ffn MOE_FFN_UP)",
                     "bound": "mfma", "achieved": up["tflops"], "peak": peak_mm, "unit": "TFLOP/s",
                     "frac": up["tflops"] / peak_mm,
                     "traffic": None if up_traffic is None else up_traffic["bytes"],
                     "traffic_detail": up_traffic,
                     "avg_ms": up["ms"], "flops_per_launch": alg["ffn_up_flops"](rows),
                     "algorithmic_bytes_per_launch": alg["ffn_up_bytes"](rows)},
        "gemm_mfma_frac": tf(gemm_flops, gemm_ms) / peak_mm,
        "stages": stages,
        "after_step": {"bias_update": {"us": bu_us, "bytes": bu_bytes, "gb_s": bu_bytes / (bu_us * 1e-6) / 1e9,
                                       "bound": "latency (one work-group)"}},
    }
    if a.backward:
        result["backward"] = backward_bench(a, cfg, layer, x, ev, torch, alg, rows)

    # the page's exposed/hidden communication model, instantiated with this
    # run's measured routed-expert throughput and MI355X xGMI link figures
    from moe_expert_routing_sqrt_amd import overlap as OV
    if not cfg.local:
        C_meas = (alg["ffn_up_flops"](rows) + alg["ffn_down_flops"](rows)) / ((st_ms["ffn_up"] + st_ms["ffn_down"]) * 1e-3)
        pts = {"ib_50GBs": 50e9, "one_xgmi_link": OV.XGMI_LINK_GBS * 1e9, "ep4_xgmi": OV.ep_bandwidth(4),
               "ep8_xgmi": OV.ep_bandwidth(8)}
        sw = {}
        for name, B in pts.items():
            r = OV.model(C_meas, B, cfg.d, cfg.d_ff, pairs=rows)
            sw[name] = {"B_GBs": B / 1e9, "t_comp_ms": r["t_comp"] * 1e3, "t_comm_ms": r["t_comm"] * 1e3,
                        "exposed_ms": r["exposed"] * 1e3, "utilization": r["utilization"],
                        "speedup_vs_serial": r["speedup"]}
        result["overlap_model"] = {
            "C_measured_tflops": C_meas / 1e12, "pairs_per_gpu": rows,
            "crossover_flops_per_byte": OV.crossover_intensity(cfg.d, cfg.d_ff),
            "crossover_bandwidth_GBs": OV.crossover_bandwidth(C_meas, cfg.d, cfg.d_ff) / 1e9,
            "points": sw,
            "one_gpu_local_exchange_ms": st_ms["dispatch"] + st_ms["combine"]}
    if a.cpu_sample > 0:
        print("cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, ex, a.cpu_sample,
                                              None if ids is None else ids.cpu().numpy())
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
