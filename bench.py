"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload v3] [--cpu-sample S]

One step = one whole layer forward (route -> dispatch -> routed expert FFN ->
shared expert -> combine) over one batch of T tokens, inputs and weights
resident in HBM.  Prints one JSON line: tokens/s for the whole step, per-stage
times from HIP events on the stream the kernels run on, the roofline of the
dominant kernel (the routed up-projection GEMM + SwiGLU), and the CPU oracle
timed on a bounded sample of the same workload.  The full default report (V3,
CPU baseline on) also runs the other workloads -- Flash, both V3 skew ranks,
the e4m3 experts, the hash router and forward + backward -- each in a child
process of its own, and adds their figures as other_workloads (--others off:
skip them).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec on 1 MI355X; GEMM MFMA % peak; route/permute GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
HASH_SEED = 7

# HBM traffic of the up-projection launch (the dominant kernel), per launch, from two
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
    # the bf16 up-projection launch with the shared expert inside it
    "v3": {"sources": ("moe_expert_routing_sqrt_amd/csrc/ffn_bf16.hip",) + _SHARED_SOURCES,
           "sources_sha256": "2f9740eafc21bbc3ef9bf932486c6418753a7510e47540fd4aeb4161d103d39e",
           "merged": True,
           "fetch_kib": 19050597.8, "fetch_scale": 1.99997,
           "write_kib": 590195.8, "write_scale": 1.0},
    # the e4m3 routed up-projection launch (the shared expert has launches of its own)
    "v3_fp8": {"sources": ("moe_expert_routing_sqrt_amd/csrc/gemm_fp8p.hip",) + _SHARED_SOURCES,
               "sources_sha256": "a0e3f39332d50afa4c778655b57283fb15a7836d79e863c8f15ee6b1b6f6c9c6",
               "merged": False,
               "fetch_kib": 10423854.1, "fetch_scale": 1.99997,
               "write_kib": 274993.2, "write_scale": 1.0},
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
    ap.add_argument("--shared", default="merged", choices=("merged", "separate"),
                    help="merged: the shared expert is one more group of the routed expert launches; "
                         "separate: a call of its own after them")
    ap.add_argument("--backward", action="store_true",
                    help="also time forward+backward steps (bf16 top-k workload) and report the backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 2 GiB copy (counter calibration for --pmc passes)")
    ap.add_argument("--overlap", action="store_true",
                    help="expert products on most CUs beside a copy of the packed rows (the exchange's "
                         "payload) on CUs reserved by stream CU masks; one JSON line")
    ap.add_argument("--reserve", type=int, default=16, help="CUs --overlap reserves for the copy (multiple of 8)")
    ap.add_argument("--others", default="auto", choices=("auto", "on", "off"),
                    help="also run the other workloads (Flash, both V3 skew ranks, e4m3, hash router, "
                         "forward + backward), each in a child process of its own, and add their figures "
                         "to the line as other_workloads; auto: only on the full default report (V3, "
                         "top-k, CPU baseline on)")
    ap.add_argument("--down-variants", action="store_true",
                    help="as --up-variants, for the down-projection (the routed rows' h against each "
                         "variant's W2 groups; one JSON line)")
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


def algorithmic(cfg, merged=False):
    """Per-launch algorithmic work of each stage: the bytes the method must move
    or the FLOPs it must compute, padding and re-reads excluded.  merged: the
    shared expert's rows are one more group of the routed expert launches."""
    T, d, E, k, d_ff = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff
    ms = T if merged else 0          # shared-expert rows inside the expert launches
    P = T * k if not cfg.local else None
    act = 4 if cfg.dtype == "f32" else 2
    # packed-row bytes: e4m3 codes plus one fp32 scale per 128 columns for fp8
    packed = d + 4 * (d // 128) if cfg.dtype == "fp8" else d * act
    wbytes = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.dtype]
    return {
        "route_flops": 2 * T * d * E,
        "route_select_bytes": T * E * 4 + E * 4 + T * k * 8 + ((T + 63) // 64) * E * 4,
        "dispatch_bytes": lambda rows: T * d * act + rows * packed + 12 * T * k,
        "ffn_up_flops": lambda rows: 4 * d * d_ff * (rows + ms),
        # rows in (packed, and the shared expert's own when merged), each
        # expert's W1/W3 once, h out (+ scales for fp8)
        "ffn_up_bytes": lambda rows: (rows + ms) * packed
        + (cfg.e_end - cfg.e_begin + (1 if merged else 0)) * 2 * d_ff * d * wbytes
        + (rows + ms) * (d_ff + 4 * (d_ff // 128) if cfg.dtype == "fp8" else d_ff * act)
        + ((cfg.e_end - cfg.e_begin + (1 if merged else 0)) * 2 * d_ff * d // (128 * 128) * 4
           if cfg.dtype == "fp8" else 0),
        "ffn_down_flops": lambda rows: 2 * d * d_ff * (rows + ms),
        "shared_flops": 0 if merged else 6 * d * d_ff * T,
        # the packed rows and (dest, w) in, the shared expert's rows in (not for
        # an expert-parallel share), the output out (a share: fp32, written)
        "combine_bytes": lambda rows: rows * d * act + 8 * T * k + (T * d * act if not cfg.local else 0)
        + T * d * (4 if cfg.local else act),
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


def traffic(cfg, up_bytes, merged):
    """Counter-measured HBM bytes per up-projection launch, or None."""
    rec = TRAFFIC.get(cfg.name)
    if rec is None or rec["sources_sha256"] != sources_digest(rec["sources"]) or rec["merged"] != merged:
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, ex, S, ids=None):
    """The oracle on the host: route and dispatch on all T tokens (logits in
    fp64 BLAS, selection and the stable permutation in numpy), the expert FFNs
    and the combine on the first S tokens (streaming one expert's weights at a
    time); each stage's seconds per token from its own token count, the layer
    rate from their sum."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import combine as OC, dispatch as OD, ffn as OF, hash_route as OH, route as OR

    S = min(S, cfg.T)
    T = cfg.T
    x_all = inp["x"].float().cpu().numpy()
    x = x_all[:S]
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

    def route_all():
        if ids is None:
            _, idx_, w_ = OR.route(x_all, wg, bias, cfg.G, cfg.M, cfg.k, cfg.gk, off)
        else:
            idx_, w_ = OH.hash_route(ids, cfg.E, cfg.k, HASH_SEED)
        return idx_, w_

    t0 = time.perf_counter()
    idx, w = route_all()
    t1 = time.perf_counter()
    _, _, _, src_all = OD.dispatch(idx, cfg.E, cfg.e_begin, cfg.e_end)
    OD.pack(x_all, src_all)
    t2 = time.perf_counter()
    # the FFN and combine on the first S tokens' pairs
    counts, offsets, dest, src = OD.dispatch(idx[:S], cfg.E, cfg.e_begin, cfg.e_end)
    xp = OD.pack(x, src)
    t3 = time.perf_counter()
    yp, _ = OF.grouped_ffn(xp, offsets, None, None, weight_fn=lambda i: (f(w13_h[i]), f(w2_h[i])))
    t4 = time.perf_counter()
    ysh = None
    if not cfg.local:
        ysh, _ = OF.expert_forward(x, f(sh13), f(sh2))
    t5 = time.perf_counter()
    if cfg.local:
        OC.combine(yp, dest, w[:S], out_init=np.zeros((S, cfg.d)))
    else:
        OC.combine(yp, dest, w[:S], ysh=ysh)
    t6 = time.perf_counter()
    per_tok = {"route": (t1 - t0) / T, "dispatch": (t2 - t1) / T, "routed_experts": (t4 - t3) / S,
               "shared_expert": (t5 - t4) / S, "combine": (t6 - t5) / S}
    ntok = {"route": T, "dispatch": T, "routed_experts": S, "shared_expert": S, "combine": S}
    for name, spt in per_tok.items():
        st[name] = {"seconds": spt * ntok[name], "tokens": ntok[name], "tokens_per_s": 1.0 / max(spt, 1e-12)}
    # route and dispatch again on one core
    with threadpool_limits(1):
        u0 = time.perf_counter()
        idx1, _ = route_all()
        u1 = time.perf_counter()
        _, _, _, src1 = OD.dispatch(idx1, cfg.E, cfg.e_begin, cfg.e_end)
        OD.pack(x_all, src1)
        u2 = time.perf_counter()
    st["route_one_core"] = {"seconds": u1 - u0, "tokens": T, "tokens_per_s": T / max(u1 - u0, 1e-9)}
    st["dispatch_one_core"] = {"seconds": u2 - u1, "tokens": T, "tokens_per_s": T / max(u2 - u1, 1e-9)}
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    total = t6 - t0
    return {"value": 1.0 / sum(per_tok.values()), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"route and dispatch on all {T} tokens; expert FFNs, shared expert and combine on "
                      f"the first {S} tokens (every routed expert they reach), fp64 numpy; value = 1 / sum "
                      f"of the stages' seconds per token; {total:.1f} s in all",
            "seconds": total, "stages": st}


def up_variants(torch, M, cfg, layer, x, ids, stage="up"):
    """The routed up-projection (stage "down": down-projection) of one
    forward, then the same packed rows split equally over the experts (every
    tile full, every expert's own weights) and given to one expert (one weight
    set), in that order: the mean of five back-to-back launches each, printed
    as one JSON line.  Three forwards first bring the clocks up."""
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
    flops = (4 if stage == "up" else 2) * cfg.d * cfg.d_ff * rows
    res = {}
    for name, off, w13, w13_s in variants:
        # the down-projection variants take W2 of the same experts (one for dense)
        w2 = layer.w2 if name != "dense" else layer.w2[:1]
        w2_s = layer.w2_s if name != "dense" else first(layer.w2_s)
        # five back-to-back launches between two events on the launch stream
        # (no host gap between them); the first (untimed) brings the clocks up
        run = lambda: M.expert_ffn(off, layer.max_rows, b["xp"], w13, w2, layer.dtype,
                                   xp_scale=b["xp_scale"], w13_scale=w13_s, w2_scale=w2_s, h=layer.h,
                                   h_scale=layer.h_s, yp=layer.yp,
                                   stages=M.MOE_FFN_UP if stage == "up" else M.MOE_FFN_DOWN)
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res[name] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12}
    print(json.dumps({f"{stage}_variants": res, "workload": workload_name(cfg), "rows": rows}), flush=True)


# the other workloads of the full report: name, bench.py arguments
OTHERS = (("flash", ["--workload", "flash"]),
          ("v3_skew_ep0", ["--workload", "v3_skew_ep0"]),
          ("v3_skew_ep63", ["--workload", "v3_skew_ep63"]),
          ("v3_fp8", ["--workload", "v3_fp8"]),
          ("v3_hash_router", ["--router", "hash"]),
          ("v3_forward_backward", ["--backward"]))


def other_workloads(steps, warmup):
    """Each other workload in a child process of its own (its own weights and
    buffers; this process's are idle meanwhile), summarised from the child's
    line."""
    out = {}
    for name, args in OTHERS:
        cmd = [sys.executable, "-u", os.path.abspath(__file__), *args, "--steps", str(steps), "--warmup",
               str(warmup), "--cpu-sample", "0", "--others", "off"]
        print(f"other workload {name} ...", file=sys.stderr, flush=True)
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        except subprocess.TimeoutExpired:
            # (a child normally takes seconds: the rest are not started)
            out[name] = {"error": "timed out after 300 s; the remaining workloads were skipped"}
            break
        line = next((l for l in reversed(r.stdout.splitlines()) if l.startswith('{"metric"')), None)
        if r.returncode != 0 or line is None:
            out[name] = {"error": f"exit status {r.returncode}", "stderr_tail": r.stderr[-400:]}
            continue
        j = json.loads(line)
        o = {"workload": j["config"]["workload"], "dtype": j["dtype"], "ms_per_step": j["ms_per_step"],
             "tokens_per_s": j["value"], "steps": j["steps"],
             "stages_ms": {k: v["ms"] for k, v in j["stages"].items()},
             "up_projection_frac_of_peak": j["roofline"]["frac"], "gemm_frac_of_peak": j["gemm_mfma_frac"]}
        for k in ("dispatch", "combine"):
            o[f"{k}_frac_hbm"] = j["stages"][k].get("frac_hbm")
        if "backward" in j:
            b = j["backward"]
            o["backward"] = {k: b[k] for k in ("steps", "fwd_bwd_ms_per_step", "fwd_bwd_tokens_per_s", "bwd_ms",
                                               "stages_ms", "routed_experts_frac_mfma")}
        out[name] = o
    return out


def cu_mask_streams(torch, n_cus, reserve):
    """Two streams that split the CUs (hipExtStreamCreateWithCUMask): the
    reserved set takes reserve/8 CUs of every XCD -- bits x*32 + j for XCD x
    under a per-XCD block numbering, and bits whose index mod 8 is x under an
    interleaved one, so it is spread evenly either way -- the other stream the
    rest.  Default priority for both."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    words = (n_cus + 31) // 32
    per = reserve // 8
    res = [0] * words
    for x in range(8):
        for j in range(per):
            bit = x * 32 + (per * x + j) % 32
            res[bit // 32] |= 1 << (bit % 32)
    rest = [(~r) & 0xFFFFFFFF for r in res]
    streams = []
    for m in (rest, res):
        h = ctypes.c_void_p()
        arr = (ctypes.c_uint32 * words)(*m)
        st = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), arr)
        if st != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({st})")
        streams.append(torch.cuda.ExternalStream(h.value))
    destroy = lambda: [hip.hipStreamDestroy(ctypes.c_void_p(st.cuda_stream)) for st in streams]
    return streams, res, destroy


def overlap(torch, M, cfg, layer, x, ids, reserve):
    """The expert products of one forward (up + SwiGLU, down; the shared expert
    inside) beside a copy of the packed rows -- the bytes an expert-parallel
    exchange moves for this GPU -- on another stream: each alone on the whole
    chip, each alone on its part of a CU split (reserve CUs for the copy, the
    rest for the products), both at once on the split, and both at once on two
    plain streams.  Mean of 5 back-to-back repetitions each; the products'
    output on the split is checked equal to the whole-chip one."""
    for _ in range(3):
        layer.forward(x, token_ids=ids)
    torch.cuda.synchronize()
    b = layer.dbufs
    payload = b["xp"]
    recv = torch.empty_like(payload)
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    (s_main, s_comm), res_mask, destroy_streams = cu_mask_streams(torch, n_cus, reserve)
    p1, p2 = torch.cuda.Stream(), torch.cuda.Stream()
    extra = None
    if layer.merge_shared:
        extra = dict(rows=layer.T, x=x, w13=layer.sh_w13, w2=layer.sh_w2, h=layer.sh_h, y=layer.ysh)

    def experts():
        for st in (M.MOE_FFN_UP, M.MOE_FFN_DOWN):
            M.expert_ffn(b["offsets"], layer.max_rows, b["xp"], layer.w13, layer.w2, layer.dtype,
                         xp_scale=b["xp_scale"], w13_scale=layer.w13_s, w2_scale=layer.w2_s, h=layer.h,
                         h_scale=layer.h_s, yp=layer.yp, stages=st, ws=layer.ffn_ws, extra=extra)

    def copy():
        recv.copy_(payload)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()

    def timed(jobs, reps=5):
        """jobs: (stream, fn) pairs started together; ms per repetition from a
        start event that every stream waits for to the last stream's end."""
        for st, fn in jobs:   # one untimed round
            with torch.cuda.stream(st):
                fn()
        torch.cuda.synchronize()
        start, ends = ev(), []
        start.record(cur)
        for st, _ in jobs:
            st.wait_event(start)
        for st, fn in jobs:
            with torch.cuda.stream(st):
                for _ in range(reps):
                    fn()
            e = ev()
            e.record(st)
            ends.append(e)
        torch.cuda.synchronize()
        return max(start.elapsed_time(e) for e in ends) / reps

    res = {}
    res["experts_whole_chip_ms"] = timed([(cur, experts)])
    y_ref = layer.yp.clone()
    res["copy_whole_chip_ms"] = timed([(cur, copy)])
    res["experts_on_split_ms"] = timed([(s_main, experts)])
    assert torch.equal(layer.yp, y_ref), "expert products on the CU split differ"
    res["copy_on_reserved_ms"] = timed([(s_comm, copy)])
    res["both_on_split_ms"] = timed([(s_main, experts), (s_comm, copy)])
    res["both_on_plain_streams_ms"] = timed([(p1, experts), (p2, copy)])
    assert torch.equal(layer.yp, y_ref)
    assert torch.equal(recv, payload)
    torch.cuda.synchronize()
    destroy_streams()
    serial = res["experts_whole_chip_ms"] + res["copy_whole_chip_ms"]
    res["serial_ms"] = serial
    res["hidden_fraction_of_copy_on_split"] = (serial - res["both_on_split_ms"]) / res["copy_whole_chip_ms"]
    # the copy's own time on its reserved CUs that the products' span covers
    res["copy_covered_on_split"] = ((res["experts_on_split_ms"] + res["copy_on_reserved_ms"] - res["both_on_split_ms"])
                                    / res["copy_on_reserved_ms"])
    res["hidden_fraction_of_copy_plain"] = (serial - res["both_on_plain_streams_ms"]) / res["copy_whole_chip_ms"]
    print(json.dumps({"overlap": res, "reserved_cus": reserve, "cus": n_cus,
                      "reserved_mask": [hex(m) for m in res_mask],
                      "payload_bytes": payload.numel() * payload.element_size(),
                      "workload": workload_name(cfg)}), flush=True)


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
                       group_topk=cfg.gk, router=a.router, hash_seed=HASH_SEED,
                       merge_shared=a.shared == "merged")
    x = inp["x"]
    ids = gen.token_ids(cfg, device=dev) if a.router == "hash" else None
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f}s: {workload_name(cfg, a.router)}", file=sys.stderr, flush=True)
    if a.up_variants or a.down_variants:
        up_variants(torch, M, cfg, layer, x, ids, "up" if a.up_variants else "down")
        return
    if a.overlap:
        overlap(torch, M, cfg, layer, x, ids, a.reserve)
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

    # route selection alone (affinities, group and expert selection, weights,
    # block histogram) from the step's logits, back to back
    sel_us = None
    if a.router == "topk":
        sel_idx, sel_w, sel_bc = (torch.empty_like(layer.idx), torch.empty_like(layer.topk_w),
                                  torch.empty_like(layer.block_counts))
        rs0, rs1 = ev(), ev()
        rs0.record()
        for _ in range(reps):
            M.route(layer.sh, None, None, layer.bias, layer.logit_offset, logits=layer.logits, logits_in=True,
                    idx=sel_idx, w=sel_w, block_counts=sel_bc)
        rs1.record()
        torch.cuda.synchronize()
        sel_us = rs0.elapsed_time(rs1) / reps * 1e3
        assert torch.equal(sel_idx, layer.idx)

    # this GPU's row of the expert-parallel send matrix: packed rows per
    # destination group (the slice of the group-ordered buffer each group's
    # owner would receive), and rows per local expert
    cnt = layer.dbufs["counts"].cpu().tolist()
    gsz = cfg.E // cfg.G
    per_group = [0] * cfg.G
    for i, c in enumerate(cnt):
        per_group[(cfg.e_begin + i) // gsz] += c
    srt = sorted(cnt)
    send_row = {"rows_per_group": per_group, "local_experts": [cfg.e_begin, cfg.e_end],
                "rows_per_expert": {"min": srt[0], "median": srt[len(srt) // 2], "max": srt[-1],
                                    "max_over_mean": srt[-1] / max(sum(srt) / len(srt), 1e-9)}}
    if len(cnt) <= 8:
        send_row["rows_per_expert"]["all"] = cnt

    names = ("route", "dispatch", "ffn_up", "ffn_down", "shared", "combine")
    st_ms = {n: sum(m[i].elapsed_time(m[i + 1]) for m in marks) / a.steps for i, n in enumerate(names)}
    rows = int(layer.dbufs["offsets"][-1].item())
    merged = bool(getattr(layer, "merge_shared", False))
    alg = algorithmic(cfg, merged)
    peak_mm = PEAK_FP8_TFLOPS if cfg.dtype == "fp8" else PEAK_BF16_TFLOPS
    tf = lambda flops, ms: flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    gbs = lambda byts, ms: byts / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    if a.router == "topk":
        sel_ms = sel_us * 1e-3
        gate_ms = max(st_ms["route"] - sel_ms, 1e-9)
        route_stage = {"ms": st_ms["route"], "gate_ms": gate_ms, "gate_tflops": tf(alg["route_flops"], gate_ms),
                       "gate_frac_mfma": tf(alg["route_flops"], gate_ms) / PEAK_BF16_TFLOPS,
                       "select_us": sel_us, "select_bytes": alg["route_select_bytes"],
                       "select_gb_s": gbs(alg["route_select_bytes"], sel_ms),
                       "select_frac_hbm": gbs(alg["route_select_bytes"], sel_ms) / PEAK_HBM_GBS,
                       "note": "gate_ms = route stage minus the selection timed alone from finished logits "
                               "(the weight planes' preparation, and in the step the summing of the split gate "
                               "product's partial products inside the selection, count with the gate product); "
                               "gate_tflops on 2*T*d*E useful flops"}
    stages = {
        "route": (route_stage
                  if a.router == "topk" else
                  {"ms": st_ms["route"], "kind": "hash router",
                   "bytes": cfg.T * 4 + cfg.T * cfg.k * 8 + ((cfg.T + 63) // 64) * cfg.E * 4}),
        "dispatch": {"ms": st_ms["dispatch"], "gb_s": gbs(alg["dispatch_bytes"](rows), st_ms["dispatch"])},
        "ffn_up": {"ms": st_ms["ffn_up"], "tflops": tf(alg["ffn_up_flops"](rows), st_ms["ffn_up"])},
        "ffn_down": {"ms": st_ms["ffn_down"], "tflops": tf(alg["ffn_down_flops"](rows), st_ms["ffn_down"])},
        "shared": ({"ms": st_ms["shared"], "merged": "the shared expert's tiles run in the ffn_up and "
                                                      "ffn_down launches (counted there)"} if merged else
                   {"ms": st_ms["shared"], "tflops": tf(alg["shared_flops"] if layer.has_shared else 0,
                                                        st_ms["shared"])}),
        "combine": {"ms": st_ms["combine"], "gb_s": gbs(alg["combine_bytes"](rows), st_ms["combine"])},
    }
    for s in ("dispatch", "combine"):
        stages[s]["frac_hbm"] = stages[s]["gb_s"] / PEAK_HBM_GBS
    for s in ("ffn_up", "ffn_down", "shared"):
        if "tflops" in stages[s]:
            stages[s]["frac_mfma"] = stages[s]["tflops"] / peak_mm
    gemm_ms = st_ms["ffn_up"] + st_ms["ffn_down"] + st_ms["shared"]
    gemm_flops = alg["ffn_up_flops"](rows) + alg["ffn_down_flops"](rows) + (alg["shared_flops"] if layer.has_shared else 0)
    up = stages["ffn_up"]
    up_traffic = traffic(cfg, alg["ffn_up_bytes"](rows), merged)
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
        "roofline": {"kernel": ("expert up-projection GEMM + SwiGLU, the routed experts and the shared expert in "
                                "one launch (moe_expert_ffn MOE_FFN_UP, shared expert as moe_ffn_extra)" if merged else
                                "routed up-projection GEMM + SwiGLU (moe_expert_ffn MOE_FFN_UP)"),
                     "bound": "mfma", "achieved": up["tflops"], "peak": peak_mm, "unit": "TFLOP/s",
                     "frac": up["tflops"] / peak_mm,
                     "traffic": None if up_traffic is None else up_traffic["bytes"],
                     "traffic_detail": up_traffic,
                     "avg_ms": up["ms"], "flops_per_launch": alg["ffn_up_flops"](rows),
                     "algorithmic_bytes_per_launch": alg["ffn_up_bytes"](rows)},
        "gemm_mfma_frac": tf(gemm_flops, gemm_ms) / peak_mm,
        "stages": stages,
        "send_matrix_row": send_row,
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
    run_others = a.others == "on" or (a.others == "auto" and a.workload == "v3" and a.router == "topk" and
                                      a.cpu_sample > 0 and not a.backward)
    if run_others:
        del layer, inp, ex, x
        torch.cuda.empty_cache()
        result["other_workloads"] = other_workloads(a.steps, a.warmup)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
