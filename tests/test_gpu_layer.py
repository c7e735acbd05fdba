"""GPU parity, end to end (S6): the whole layer through MoELayer (the launch
configuration the benchmark times) against the oracle, each side forming its
own logits.

The GPU's logits differ from the oracle's fp64-formed ones by rounding (within
1e-5 per row), so a token whose selection sits on a near-tie may flip.  Every
flipped token is listed with its decision gaps under the oracle's logits (the
smallest gap between consecutive biased affinities among the first k+1
eligible experts, and the gap between the M-th and (M+1)-th group score) and
must have a gap the token's measured logit difference can close: at most
0.35 (the largest slope of sqrt(softplus)) times max |dL| per affinity, plus
a few fp32 ulps of rounding (group scores: group_topk times that).  The output
is then compared with the oracle on the tokens whose routing matches, and
again with the oracle's routing substituted (the GPU routing from the oracle's
logits, which is bit-exact), which also covers the flipped tokens."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from oracle import combine as OC, dispatch as OD, ffn as OF, route as OR

from gpu_util import dev_f32, host, moe_shape, need_gpu, rel_max_err, router_inputs

pytestmark = pytest.mark.gpu

SLOPE = 0.35   # max over l of d sqrt(softplus(l)) / dl (0.32 near l = 1.2)


def _layer(cfg, inp, ex):
    return M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                      inp["bias"], ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"],
                      logit_offset=inp["logit_offset"], e_begin=cfg.e_begin, e_end=cfg.e_end,
                      group_topk=cfg.gk)


def _decision_gaps(L_row, o, cfg):
    """(expert gap, group gap) of one token under the oracle's logits."""
    s, b = OR.scores(L_row[None], o["bias"], o["offset"])
    gs = OR.group_scores(b, cfg.G, cfg.gk)[0].astype(np.float64)
    order = np.argsort(-gs, kind="stable")
    gap_g = float(gs[order[cfg.M - 1]] - gs[order[cfg.M]]) if cfg.M < cfg.G else np.inf
    gsz = cfg.E // cfg.G
    keep = np.zeros(cfg.E, bool)
    for g in order[:cfg.M]:
        keep[g * gsz:(g + 1) * gsz] = True
    be = np.sort(b[0][keep].astype(np.float64))[::-1][: cfg.k + 1]
    gap_e = float(np.min(be[:-1] - be[1:])) if be.size > 1 else np.inf
    return gap_e, gap_g, float(np.abs(b).max())


def check_flips(idx_gpu, L_gpu, o, cfg):
    """Lists and checks every token whose GPU selection differs from the
    oracle's; returns their indices."""
    bad = np.nonzero((idx_gpu != o["idx"]).any(1))[0]
    L_o = o["L"]
    for t in bad:
        dl = float(np.abs(L_gpu[t].astype(np.float64) - L_o[t]).max())
        gap_e, gap_g, bmax = _decision_gaps(L_o[t], o, cfg)
        ulp = float(np.spacing(np.float32(bmax)))
        allow_e = SLOPE * dl + 4 * ulp
        allow_g = cfg.gk * SLOPE * dl + 8 * ulp
        print(f"  flipped token {t}: oracle {o['idx'][t].tolist()} gpu {idx_gpu[t].tolist()}; "
              f"max|dL| {dl:.2e}; expert gap {gap_e:.2e} (allowed {allow_e:.2e}), "
              f"group gap {gap_g:.2e} (allowed {allow_g:.2e})")
        assert gap_e <= allow_e or gap_g <= allow_g, t
    return bad


def _oracle_tokens(cfg, o, ex, toks, dev):
    """The oracle's layer output for the listed tokens (fp64), streaming one
    expert's weights at a time through a thread pool."""
    toks = list(toks)
    pos = {t: i for i, t in enumerate(toks)}
    users = {}
    for t in toks:
        for j in range(cfg.k):
            e = int(o["idx"][t, j])
            if cfg.e_begin <= e < cfg.e_end:
                users.setdefault(e, []).append((pos[t], float(o["w"][t, j])))
    xs = o["x"][toks]

    def part(item):
        e, uses = item
        if e < 0:
            w13, w2 = host(ex["sh_w13"][0]), host(ex["sh_w2"][0])
        else:
            w13, w2 = host(ex["w13"][e - cfg.e_begin]), host(ex["w2"][e - cfg.e_begin])
        rows = [i for i, _ in uses]
        y, _ = OF.expert_forward(xs[rows], w13, w2)
        return rows, np.array([w for _, w in uses])[:, None] * y

    work = sorted(users.items())
    if not cfg.local:
        work.append((-1, [(i, 1.0) for i in range(len(toks))]))
    out = np.zeros((len(toks), cfg.d))
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    # (one BLAS thread per worker: the pool is the parallelism)
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers) as pool:
        for i, (rows, y) in enumerate(pool.map(part, work)):
            np.add.at(out, rows, y)
            if i % 32 == 31:
                print(f"  oracle: {i + 1} of {len(work)} experts", flush=True)
    return out


@pytest.mark.parametrize("name", ["tiny", "flash"])
def test_layer_end_to_end(name):
    dev = need_gpu()
    cfg, inp, o = router_inputs(name)
    print(f"layer S6 {name}", flush=True)
    ex = gen.make_experts(cfg, device=dev)
    layer = _layer(cfg, inp, ex)
    out = host(layer.forward(inp["x"]))
    torch.cuda.synchronize()
    bad = check_flips(host(layer.idx), host(layer.logits), o, cfg)
    print(f"  routing flips vs oracle logits: {len(bad)} of {cfg.T}")
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    yp, _ = OF.grouped_ffn(OD.pack(o["x"], src), offsets, host(ex["w13"]), host(ex["w2"]))
    ysh, _ = OF.expert_forward(o["x"], host(ex["sh_w13"][0]), host(ex["sh_w2"][0]))
    ref = OC.combine(yp, dest, o["w"], ysh=ysh)
    ok = np.ones(cfg.T, bool)
    ok[bad] = False
    err = rel_max_err(out[ok], ref[ok])
    print(f"  rel max err on matched tokens {err:.3e}")
    assert err <= (1e-5 if cfg.dtype == "f32" else 2e-2)


def _forward_with_oracle_routing(layer, cfg, o, x, dev):
    """The layer's dispatch, experts and combine on the oracle's routing (the
    GPU routes from the oracle's logits, bit-exact)."""
    sh = moe_shape(cfg)
    _, idx, w, bc = M.route(sh, None, None, dev_f32(o["bias"], dev),
                            None if o["offset"] is None else dev_f32(o["offset"], dev),
                            logits=dev_f32(o["L"], dev), logits_in=True)
    b = M.dispatch(sh, idx, bc, x, cfg.e_begin, cfg.e_end)
    yp, _, _ = M.expert_ffn(b["offsets"], cfg.T * cfg.k, b["xp"], layer.w13, layer.w2)
    ysh = None
    if layer.has_shared:
        ysh, _, _ = M.expert_ffn(layer.sh_offsets, cfg.T, x, layer.sh_w13, layer.sh_w2)
    if cfg.local:
        out = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device=dev)
        M.combine(sh, b["dest"], w, yp, None, out=out, accumulate=True)
    else:
        out = M.combine(sh, b["dest"], w, yp, ysh)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), o["idx"])
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T", [("v3", None), ("v3_skew_ep0", None), ("v3_skew_ep63", None), ("v3", 65536)])
def test_layer_v3_sampled_tokens(name, T):
    """Full V3 size (and one expert-parallel rank's share under skew; and 4x
    the tokens, 524288 routed rows): 1024 sampled tokens plus the last one; the
    flipped tokens are listed and checked, the matched ones compared, and all
    of them compared again with the oracle's routing substituted."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    print(f"layer S6 {name} (sampled tokens)", flush=True)
    ex = gen.make_experts(cfg, device=dev)
    layer = _layer(cfg, inp, ex)
    out_d = layer.forward(inp["x"])
    torch.cuda.synchronize()
    bad = check_flips(host(layer.idx), host(layer.logits), o, cfg)
    print(f"  routing flips vs oracle logits: {len(bad)} of {cfg.T}")
    assert len(bad) <= cfg.T // 1000
    if cfg.local:
        counts = np.bincount(o["idx"].ravel(), minlength=cfg.E)[cfg.e_begin:cfg.e_end]
        print(f"  local rows per expert {counts.tolist()}")
    rng = np.random.default_rng(0)
    sample = sorted(set(rng.choice(cfg.T, 1024, replace=False).tolist()) | {cfg.T - 1})
    matched = [t for t in sample if t not in set(bad.tolist())]
    assert len(matched) >= 1000
    with_flips = sorted(set(sample) | set(bad.tolist()))
    ref = _oracle_tokens(cfg, o, ex, with_flips, dev)
    row = {t: i for i, t in enumerate(with_flips)}
    got = host(out_d[torch.tensor(matched, device=dev)])
    err = rel_max_err(got, ref[[row[t] for t in matched]])
    print(f"  {len(matched)} matched tokens: rel max err {err:.3e}")
    assert err <= 2e-2
    out2 = _forward_with_oracle_routing(layer, cfg, o, inp["x"], dev)
    got2 = host(out2[torch.tensor(with_flips, device=dev)])
    err2 = rel_max_err(got2, ref)
    print(f"  oracle routing substituted, {len(with_flips)} tokens ({len(bad)} flipped): rel max err {err2:.3e}")
    assert err2 <= 2e-2
    del layer, ex
    torch.cuda.empty_cache()


def test_layer_local_share_twice():
    """A local expert range forward into the layer's own fp32 output, twice in
    a row, the buffer holding NaN before the first: both results equal the
    oracle's share (the layer writes every row of its own output, 0 where no
    local expert was chosen).  Into a caller's fp32 buffer the share is added
    to what the buffer holds."""
    dev = need_gpu()
    cfg = C.get("v3_skew_ep0").with_(T=2048, d=512, d_ff=256)
    print(f"layer local share twice T={cfg.T} d={cfg.d}", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    layer = _layer(cfg, inp, ex)
    L = OR.gate_logits(host(inp["x"]), host(inp["w_gate"]))
    o = {"bias": host(inp["bias"]), "offset": host(inp["logit_offset"])}
    layer.out.fill_(float("nan"))
    first = host(layer.forward(inp["x"])).copy()
    second = host(layer.forward(inp["x"]))
    acc = torch.full((cfg.T, cfg.d), 1.0, dtype=torch.float32, device=dev)
    added = host(layer.forward(inp["x"], out=acc))
    torch.cuda.synchronize()
    idx_g, w_g = host(layer.idx), host(layer.topk_w)
    # the oracle's share for the GPU's own routing (any flips are then shared)
    gi, gw = OR.route_from_logits(host(layer.logits), o["bias"], cfg.G, cfg.M, cfg.k, cfg.gk, o["offset"])
    assert np.array_equal(gi, idx_g)
    counts, offsets, dest, src = OD.dispatch(gi, cfg.E, cfg.e_begin, cfg.e_end)
    yp, _ = OF.grouped_ffn(OD.pack(host(inp["x"]), src), offsets, host(ex["w13"]), host(ex["w2"]))
    ref = OC.combine(yp, dest, gw, out_init=np.zeros((cfg.T, cfg.d)))
    print(f"  local rows per expert {counts.tolist()}")
    assert rel_max_err(first, ref) <= 2e-2
    assert np.array_equal(first, second)
    # the add starts from the buffer's value, so it rounds differently from
    # 1 + share: a few fp32 ulps of the larger term
    scale = 1.0 + float(np.abs(first).max())
    assert float(np.abs(added.astype(np.float64) - (1.0 + first.astype(np.float64))).max()) <= 1e-5 * scale
