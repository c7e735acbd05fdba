"""GPU parity: the MoE layer backward against the oracle (oracle/backward.py).

Stage by stage at small ragged sizes, end to end through the stage calls
(routing driven by the oracle's logits, so the selection is identical), and at
the 16K-token size a sampled expert and a 256-token gradient subset (dx,
d_topk_w, dW_g, two experts' weight gradients).  Bars: combine's d_yp within one bf16
ulp of the fp64 product (it is one rounded product), fp32 sums within 1e-5
relative, bf16 expert products within 2e-2 relative (max over the tensor,
relative to its largest entry), as for the forward FFN."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from oracle import backward as OB, combine as OC, dispatch as OD, ffn as OF, route as OR

from gpu_util import dev_f32, dev_i32, expert_host, host, need_gpu, rel_max_err

pytestmark = pytest.mark.gpu


def _bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# 300 small experts (0..70 rows, a few empty): 600 weight-gradient tiles of
# one or two K steps, so each persistent work-group runs a stream of several
# tiles of different experts
MANY_SMALL = [(i * 37) % 71 for i in range(300)]


@pytest.mark.parametrize("counts,d,d_ff", [([0, 1, 300, 257, 129], 512, 256), ([700], 256, 512),
                                           ([64, 0, 0, 200], 256, 256), (MANY_SMALL, 256, 256)])
def test_expert_ffn_backward_grouped(counts, d, d_ff):
    dev = need_gpu()
    print(f"ffn backward counts={counts if len(counts) < 10 else f'{len(counts)} groups'} d={d} d_ff={d_ff}",
          flush=True)
    rng = np.random.default_rng(sum(counts) + d + d_ff)
    n, rows = len(counts), int(sum(counts))
    xp = _bf16(rng.normal(size=(rows, d)), dev)
    w13 = _bf16(rng.normal(size=(n, 2 * d_ff, d)) * 0.05, dev)
    w2 = _bf16(rng.normal(size=(n, d, d_ff)) * 0.05, dev)
    dy = _bf16(rng.normal(size=(rows, d)), dev)
    off = _offsets(counts)
    b = M.expert_ffn_backward(dev_i32(off, dev), rows, xp, w13, w2, dy)
    torch.cuda.synchronize()
    r_dx, r_dw13, r_dw2 = OB.grouped_ffn_backward(host(xp), off, host(w13), host(w2), host(dy))
    assert rel_max_err(host(b["d_xp"])[:rows], r_dx) <= 2e-2
    for e in range(n):
        if counts[e] == 0:
            assert np.all(host(b["dw13"][e]) == 0) and np.all(host(b["dw2"][e]) == 0)
            continue
        assert rel_max_err(host(b["dw13"][e]), r_dw13[e]) <= 2e-2, e
        assert rel_max_err(host(b["dw2"][e]), r_dw2[e]) <= 2e-2, e


def test_expert_ffn_backward_one_group_without_offsets():
    dev = need_gpu()
    rng = np.random.default_rng(7)
    rows, d, d_ff = 333, 256, 256
    x = _bf16(rng.normal(size=(rows, d)), dev)
    w13 = _bf16(rng.normal(size=(1, 2 * d_ff, d)) * 0.05, dev)
    w2 = _bf16(rng.normal(size=(1, d, d_ff)) * 0.05, dev)
    g = _bf16(rng.normal(size=(rows, d)), dev)
    b = M.expert_ffn_backward(None, rows, x, w13, w2, g)
    torch.cuda.synchronize()
    r_dx, r_dw13, r_dw2 = OB.expert_backward(host(x), host(w13[0]), host(w2[0]), host(g))
    assert rel_max_err(host(b["d_xp"]), r_dx) <= 2e-2
    assert rel_max_err(host(b["dw13"][0]), r_dw13) <= 2e-2
    assert rel_max_err(host(b["dw2"][0]), r_dw2) <= 2e-2


def _routing(rng, T, E, k, local=None):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    e0, e1 = (0, E) if local is None else local
    counts, offsets, dest, src = OD.dispatch(idx, E, e0, e1)
    return idx, offsets, dest, src


@pytest.mark.parametrize("y_dt,g_dt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                       (torch.bfloat16, torch.float32)])
def test_combine_backward(y_dt, g_dt):
    dev = need_gpu()
    rng = np.random.default_rng(3)
    T, E, k, d = 300, 32, 6, 512
    idx, offsets, dest, src = _routing(rng, T, E, k, local=(4, 20))   # some slots not local
    rows = int(offsets[-1])
    yp = torch.from_numpy(rng.normal(size=(rows, d)).astype(np.float32)).to(dev).to(y_dt)
    g = torch.from_numpy(rng.normal(size=(T, d)).astype(np.float32)).to(dev).to(g_dt)
    w = rng.uniform(0.05, 0.5, size=(T, k)).astype(np.float32)
    sh = M.shape(T, d, E, 4, 2, k, 256, 3)
    d_yp, d_w = M.combine_backward(sh, dev_i32(dest, dev), dev_f32(w, dev), yp, g)
    torch.cuda.synchronize()
    r_dyp, r_dw = OB.combine_backward(host(g), host(yp), dest, w, rows)
    got = host(d_yp)
    ulp = np.abs(r_dyp) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(got - r_dyp) <= ulp)
    assert np.abs(host(d_w) - r_dw).max() <= 1e-5 * np.abs(r_dw).max()
    assert np.all(host(d_w)[dest < 0] == 0)


def test_dispatch_backward():
    dev = need_gpu()
    rng = np.random.default_rng(4)
    T, E, k, d = 257, 16, 4, 256
    idx, offsets, dest, src = _routing(rng, T, E, k, local=(0, 12))
    rows = int(offsets[-1])
    dxp = _bf16(rng.normal(size=(rows, d)), dev)
    extra = _bf16(rng.normal(size=(T, d)), dev)
    sh = M.shape(T, d, E, 4, 2, k, 256, 2)
    dx = M.dispatch_backward(sh, dev_i32(dest, dev), dxp, d_extra=extra)
    torch.cuda.synchronize()
    ref = OB.dispatch_backward(host(dxp), dest, T) + host(extra)
    assert np.abs(host(dx) - ref).max() <= 1e-6 * np.abs(ref).max()
    base = dx.clone()
    M.dispatch_backward(sh, dev_i32(dest, dev), dxp, dx=dx, accumulate=True)
    torch.cuda.synchronize()
    assert np.abs(host(dx) - (host(base) + OB.dispatch_backward(host(dxp), dest, T))).max() <= 1e-6 * np.abs(ref).max()


@pytest.mark.parametrize("with_offset,T,x_f32", [(False, 300, False), (True, 300, False), (False, 4100, False),
                                                 (False, 4100, True), (True, 300, True)])
def test_route_backward(with_offset, T, x_f32):
    """bf16 x: the matrix-core products over three bf16 planes per fp32
    operand (T = 4100: two row splits of dW_g, the second ragged); fp32 x: the
    vector products (T = 4100: four K parts of the workspace)."""
    dev = need_gpu()
    print(f"route backward offset={with_offset} T={T} x_f32={x_f32}", flush=True)
    rng = np.random.default_rng(5 + with_offset + T)
    E, k, d = 64, 6, 512
    x = _bf16(rng.normal(size=(T, d)), dev)
    if x_f32:
        x = x.float()
    wg = (rng.normal(size=(d, E)) * 0.02).astype(np.float32)
    L = (rng.normal(size=(T, E)) * 3).astype(np.float32)
    L.reshape(-1)[:6] = [0.0, -40.0, 40.0, 1e-6, -1e-6, 88.0]
    off = (rng.uniform(-1, 1, size=E).astype(np.float32)) if with_offset else None
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[0] = np.arange(k)                                  # the special logits are selected
    dw = rng.normal(size=(T, k)).astype(np.float32)
    dx0 = rng.normal(size=(T, d)).astype(np.float32)
    sh = M.shape(T, d, E, 8, 4, k, 256, 2)
    dx = dev_f32(dx0, dev)
    dL, dWg = M.route_backward(sh, x, dev_f32(wg, dev), dev_f32(L, dev), dev_i32(idx, dev), dev_f32(dw, dev), dx,
                               logit_offset=None if off is None else dev_f32(off, dev))
    torch.cuda.synchronize()
    Lr = L if off is None else (L + off[None, :]).astype(np.float32)    # the routed logits, in fp32
    r_dx, r_dWg, r_dL = OB.gate_backward(host(x), wg, Lr, idx, dw)
    assert np.abs(host(dL) - r_dL).max() <= 1e-5 * np.abs(r_dL).max()
    assert np.all(host(dL)[r_dL == 0] == 0)
    assert np.abs(host(dx) - (dx0 + r_dx)).max() <= 1e-5 * np.abs(r_dx).max() + 1e-6 * np.abs(dx0).max()
    assert np.abs(host(dWg) - r_dWg).max() <= 1e-5 * np.abs(r_dWg).max()


def _small_cfg():
    return C.get("flash").with_(T=512, d=512, E=16, G=4, k=4, M=2, d_ff=256)


def test_layer_backward_end_to_end():
    """Forward and backward through the stage calls, routing from the oracle's
    logits (identical selection), all gradients against the oracle."""
    dev = need_gpu()
    cfg = _small_cfg()
    print(f"backward end to end T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff}", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    x, xh = inp["x"], host(inp["x"])
    wg = host(inp["w_gate"])
    bias = host(inp["bias"])
    L = OR.gate_logits(xh, wg)
    ridx, rw = OR.route_from_logits(L, bias, cfg.G, cfg.M, cfg.k, cfg.gk)
    sh = M.shape(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.gk)
    Ld = dev_f32(L, dev)
    _, idx, w, bc = M.route(sh, None, None, inp["bias"], None, logits=Ld, logits_in=True)
    b = M.dispatch(sh, idx, bc, x)
    yp, h, _ = M.expert_ffn(b["offsets"], cfg.T * cfg.k, b["xp"], ex["w13"], ex["w2"])
    rng = np.random.default_rng(9)
    g = _bf16(rng.normal(size=(cfg.T, cfg.d)), dev)
    d_yp, d_w = M.combine_backward(sh, b["dest"], w, yp, g)
    r = M.expert_ffn_backward(b["offsets"], cfg.T * cfg.k, b["xp"], ex["w13"], ex["w2"], d_yp)
    s = M.expert_ffn_backward(None, cfg.T, x, ex["sh_w13"], ex["sh_w2"], g)
    dx = M.dispatch_backward(sh, b["dest"], r["d_xp"], d_extra=s["d_xp"])
    dL, dWg = M.route_backward(sh, x, inp["w_gate"], Ld, idx, d_w, dx)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), ridx)

    # oracle
    counts, offsets, dest, src = OD.dispatch(ridx, cfg.E)
    xp = OD.pack(xh, src)
    w13, w2 = host(ex["w13"]), host(ex["w2"])
    ryp, _ = OF.grouped_ffn(xp, offsets, w13, w2)
    gh = host(g)
    r_dyp, r_dw = OB.combine_backward(gh, ryp, dest, rw, int(offsets[-1]))
    r_dxp, r_dw13, r_dw2 = OB.grouped_ffn_backward(xp, offsets, w13, w2, r_dyp)
    r_dxs, r_ds13, r_ds2 = OB.expert_backward(xh, host(ex["sh_w13"][0]), host(ex["sh_w2"][0]), gh)
    r_dxg, r_dWg, r_dL = OB.gate_backward(xh, wg, L, ridx, r_dw)
    r_dx = OB.dispatch_backward(r_dxp, dest, cfg.T) + r_dxs + r_dxg
    errs = {"dx": rel_max_err(host(dx), r_dx), "dw13": rel_max_err(host(r["dw13"]), r_dw13),
            "dw2": rel_max_err(host(r["dw2"]), r_dw2), "dsh13": rel_max_err(host(s["dw13"][0]), r_ds13),
            "dsh2": rel_max_err(host(s["dw2"][0]), r_ds2), "dWg": rel_max_err(host(dWg), r_dWg),
            "d_w": rel_max_err(host(d_w), r_dw)}
    print("  ", {k_: f"{v:.2e}" for k_, v in errs.items()})
    for k_, v in errs.items():
        assert v <= 2e-2, (k_, v)


def test_layer_backward_v3_sampled_expert():
    """16K-token size: routed expert backward of one sampled expert (112-step
    dgrad K loops, wgrad over its ~500 rows) against the oracle."""
    dev = need_gpu()
    cfg = C.get("v3")
    print("backward v3 sampled expert", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    xh = host(inp["x"])
    L = OR.gate_logits(xh, host(inp["w_gate"]))
    ridx, rw = OR.route_from_logits(L, host(inp["bias"]), cfg.G, cfg.M, cfg.k, cfg.gk)
    sh = M.shape(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.gk)
    _, idx, w, bc = M.route(sh, None, None, inp["bias"], None, logits=dev_f32(L, dev), logits_in=True)
    b = M.dispatch(sh, idx, bc, inp["x"])
    rows = cfg.T * cfg.k
    yp, h, _ = M.expert_ffn(b["offsets"], rows, b["xp"], ex["w13"], ex["w2"])
    g = gen.normal((cfg.T, cfg.d), 1.0, dev, 0, 99).to(torch.bfloat16)
    d_yp, d_w = M.combine_backward(sh, b["dest"], w, yp, g)
    r = M.expert_ffn_backward(b["offsets"], rows, b["xp"], ex["w13"], ex["w2"], d_yp)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), ridx)
    e = 77
    toks = np.nonzero((ridx == e).any(axis=1))[0]                  # token order = row order
    slot = np.array([int(np.nonzero(ridx[t] == e)[0][0]) for t in toks])
    off = host(b["offsets"])
    lo, hi = int(off[e]), int(off[e + 1])
    assert hi - lo == toks.size
    w13_e, w2_e = host(ex["w13"][e]), host(ex["w2"][e])
    # the expert's upstream gradient rows: bf16(w * g), as the combine backward rounds them
    dy = host(d_yp[lo:hi])
    ref_dy = rw[toks, slot][:, None].astype(np.float64) * host(g)[toks]
    assert np.all(np.abs(dy - ref_dy) <= np.abs(ref_dy) * 2.0 ** -8 + 1e-30)
    r_dx, r_dw13, r_dw2 = OB.expert_backward(xh[toks], w13_e, w2_e, dy)
    errs = (rel_max_err(host(r["d_xp"][lo:hi]), r_dx), rel_max_err(host(r["dw13"][e]), r_dw13),
            rel_max_err(host(r["dw2"][e]), r_dw2))
    print(f"  expert {e}: {hi - lo} rows, errors {errs}")
    assert max(errs) <= 2e-2
    del ex, r, b
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_layer_backward_v3_token_subset():
    """16K-token size, the gradient of a loss that depends on 256 sampled
    tokens only (grad_out zero on every other token), through the stage calls
    with the oracle's routing: dx of every token (exactly zero outside the
    sample), d_topk_w and dx of the sample, dW_g, and the weight gradients of
    the two experts the sample reaches most, against the oracle run on the
    sample alone."""
    dev = need_gpu()
    cfg = C.get("v3")
    print("backward v3 token subset", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    x = inp["x"]
    xh, wg = host(x), host(inp["w_gate"])
    L = OR.gate_logits(xh, wg)
    ridx, rw = OR.route_from_logits(L, host(inp["bias"]), cfg.G, cfg.M, cfg.k, cfg.gk)
    sh = M.shape(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.gk)
    Ld = dev_f32(L, dev)
    _, idx, w, bc = M.route(sh, None, None, inp["bias"], None, logits=Ld, logits_in=True)
    b = M.dispatch(sh, idx, bc, x)
    rows = cfg.T * cfg.k
    yp, _, _ = M.expert_ffn(b["offsets"], rows, b["xp"], ex["w13"], ex["w2"])
    S = np.sort(np.random.default_rng(3).choice(cfg.T, 256, replace=False))
    mask = torch.zeros((cfg.T, 1), device=dev)
    mask[torch.from_numpy(S).to(dev)] = 1.0
    g = (gen.normal((cfg.T, cfg.d), 1.0, dev, 0, 98) * mask).to(torch.bfloat16)
    d_yp, d_w = M.combine_backward(sh, b["dest"], w, yp, g)
    r = M.expert_ffn_backward(b["offsets"], rows, b["xp"], ex["w13"], ex["w2"], d_yp)
    s = M.expert_ffn_backward(None, cfg.T, x, ex["sh_w13"], ex["sh_w2"], g)
    dx = M.dispatch_backward(sh, b["dest"], r["d_xp"], d_extra=s["d_xp"])
    _, dWg = M.route_backward(sh, x, inp["w_gate"], Ld, idx, d_w, dx)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), ridx)
    dx_h = host(dx)
    outside = np.ones(cfg.T, bool)
    outside[S] = False
    assert np.all(dx_h[outside] == 0.0)

    # oracle on the sample, one expert at a time
    xs, gs = xh[S], host(g)[S]
    users = {}
    for i, t in enumerate(S):
        for j in range(cfg.k):
            users.setdefault(int(ridx[t, j]), []).append((i, j))
    top2 = sorted(users, key=lambda e: (-len(users[e]), e))[:2]

    def part(item):
        e, uses = item
        w13, w2 = host(ex["w13"][e]), host(ex["w2"][e])
        ii = [i for i, _ in uses]
        wj = np.array([float(rw[S[i], j]) for i, j in uses])[:, None]
        y, _ = OF.expert_forward(xs[ii], w13, w2)
        d_wj = np.sum(gs[ii].astype(np.float64) * y, axis=1)            # <g_t, y_e(x_t)>
        dX, dW13, dW2 = OB.expert_backward(xs[ii], w13, w2, wj * gs[ii])
        return e, uses, d_wj, dX, (dW13, dW2) if e in top2 else None

    r_dw = np.zeros((S.size, cfg.k))
    r_dx = np.zeros((S.size, cfg.d))
    r_wg = {}
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    # (one BLAS thread per worker: the pool is the parallelism)
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers) as pool:
        for n_done, (e, uses, d_wj, dX, wgrads) in enumerate(pool.map(part, sorted(users.items()))):
            if n_done % 32 == 31:
                print(f"  oracle: {n_done + 1} of {len(users)} experts", flush=True)
            for (i, j), v in zip(uses, d_wj):
                r_dw[i, j] = v
            np.add.at(r_dx, [i for i, _ in uses], dX)
            if wgrads is not None:
                r_wg[e] = wgrads
    dXs, _, _ = OB.expert_backward(xs, host(ex["sh_w13"][0]), host(ex["sh_w2"][0]), gs)
    r_dxg, r_dWg, _ = OB.gate_backward(xs, wg, L[S], ridx[S], r_dw)
    r_dx = r_dx + dXs + r_dxg
    errs = {"dx": rel_max_err(dx_h[S], r_dx), "d_w": rel_max_err(host(d_w)[S], r_dw),
            "dWg": rel_max_err(host(dWg), r_dWg)}
    for e in top2:
        errs[f"dw13[{e}]"] = rel_max_err(host(r["dw13"][e]), r_wg[e][0])
        errs[f"dw2[{e}]"] = rel_max_err(host(r["dw2"][e]), r_wg[e][1])
    print(f"  {S.size} tokens reach {len(users)} experts;", {k_: f"{v:.2e}" for k_, v in errs.items()})
    for k_, v in errs.items():
        assert v <= 2e-2, (k_, v)
    del ex, r, s, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("counts", [[0, 1, 300, 257, 129], None])
def test_train_forward_keeps_preactivations(counts):
    """expert_ffn_train: h and yp bit-identical to expert_ffn; its [a | u] equals
    the backward's recomputation bit for bit (same K order), so the backward
    with the saved values equals the one that recomputes; [a | u] against the
    oracle's fp64 products within one bf16 rounding."""
    dev = need_gpu()
    rng = np.random.default_rng(21)
    d, d_ff = 512, 256
    rows = 700 if counts is None else int(sum(counts))
    n = 1 if counts is None else len(counts)
    off = None if counts is None else dev_i32(_offsets(counts), dev)
    xp = _bf16(rng.normal(size=(rows, d)), dev)
    w13 = _bf16(rng.normal(size=(n, 2 * d_ff, d)) * 0.05, dev)
    w2 = _bf16(rng.normal(size=(n, d, d_ff)) * 0.05, dev)
    dy = _bf16(rng.normal(size=(rows, d)), dev)
    offs = off if off is not None else dev_i32(np.array([0, rows]), dev)
    yp_ref, h_ref, _ = M.expert_ffn(offs, rows, xp, w13, w2)
    ws = {}
    h = torch.empty_like(h_ref)
    yp = torch.empty_like(yp_ref)
    M.expert_ffn_train(off, rows, xp, w13, w2, h, yp, ws)
    au_saved = ws["au"].clone()
    b1 = M.expert_ffn_backward(off, rows, xp, w13, w2, dy, ws, au_saved=True)
    out1 = {k_: b1[k_].clone() for k_ in ("d_xp", "dw13", "dw2")}
    b2 = M.expert_ffn_backward(off, rows, xp, w13, w2, dy, {})
    torch.cuda.synchronize()
    assert torch.equal(h[:rows], h_ref[:rows]) and torch.equal(yp[:rows], yp_ref[:rows])
    assert torch.equal(au_saved[:rows], b2["au"][:rows])
    for k_ in out1:
        assert torch.equal(out1[k_], b2[k_]), k_
    # [a | u] against fp64 products
    offs_h = _offsets(counts) if counts is not None else np.array([0, rows])
    xh, w13h = host(xp), host(w13)
    for e in range(n):
        lo, hi = int(offs_h[e]), int(offs_h[e + 1])
        if hi == lo:
            continue
        ref = xh[lo:hi].astype(np.float64) @ w13h[e].astype(np.float64).T
        got = host(au_saved[lo:hi])
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6 * np.abs(ref).max()), e


def test_layer_save_for_backward_matches():
    dev = need_gpu()
    cfg = _small_cfg()
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"], inp["bias"],
                       ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"], group_topk=cfg.gk)
    g = _bf16(np.random.default_rng(2).normal(size=(cfg.T, cfg.d)), dev)
    out_a = layer.forward(inp["x"]).clone()
    ga = {k_: v.clone() for k_, v in layer.backward(inp["x"], g).items()}
    out_b = layer.forward(inp["x"], save_for_backward=True).clone()
    gb = layer.backward(inp["x"], g)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    for k_ in ga:
        assert torch.equal(ga[k_], gb[k_]), k_
