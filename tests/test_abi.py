"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, its constants match the header, and bad arguments are
rejected on the host before anything is launched."""
import ctypes
import re

import pytest

from moe_expert_routing_sqrt_amd import _lib

L = _lib.load()


def test_exports_every_declared_function():
    names = _lib.header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"binding lacks a signature for {n}"
    assert sorted(_lib.SIGNATURES) == names


def test_constants_match_header():
    text = open(_lib.HEADER).read()
    defs = dict(re.findall(r"#define\s+(MOE_\w+)\s+\(?(-?\d+)\)?", text))
    for name, val in defs.items():
        if hasattr(_lib, name):
            assert getattr(_lib, name) == int(val), name
    assert L.moe_abi_version() == int(defs["MOE_ABI_VERSION"])


def test_shape_struct_layout():
    assert ctypes.sizeof(_lib.MoeShape) == 8 + 7 * 4 + 4  # int64 + 7 int32, padded to 8
    assert _lib.MoeShape.d.offset == 8


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert L.moe_status_str(st)
    assert L.moe_status_str(99) == b"unknown status"


def _sh(T=16, d=64, E=16, G=4, M=2, k=4, gk=2, d_ff=32):
    return _lib.MoeShape(T, d, E, G, M, k, gk, d_ff)


FAKE = 0x1000  # never dereferenced: every case below fails its host-side check


@pytest.mark.parametrize("bad", [
    dict(E=15), dict(G=0), dict(M=5), dict(k=9), dict(gk=5), dict(T=-1), dict(d=0), dict(d_ff=0),
    dict(E=16, G=4, M=1, k=5),
])
def test_route_rejects_bad_shapes(bad):
    sh = _sh(**bad)
    st = L.moe_route(ctypes.byref(sh), FAKE, _lib.MOE_BF16, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0,
                     FAKE, 1 << 30, None)
    assert st == _lib.MOE_ERR_INVALID_ARG


def _route(sh, x=FAKE, xdt=1, wg=FAKE, bias=FAKE, logits=FAKE, flags=0, ws=FAKE, wsb=1 << 30):
    return L.moe_route(sh, x, xdt, wg, bias, None, logits, FAKE, FAKE, FAKE, flags, ws, wsb, None)


def test_route_rejects_null_and_flags():
    sh = ctypes.byref(_sh())
    assert _route(None) == -1
    assert _route(sh, bias=None) == -1
    assert _route(sh, x=None) == -1
    assert _route(sh, wg=None) == -1
    assert _route(sh, flags=4) == -1
    assert _route(sh, xdt=7) == -1
    assert _route(sh, logits=None, flags=_lib.MOE_ROUTE_LOGITS_IN) == -1


def test_route_workspace():
    s = _sh(T=100, d=64, E=16)
    sh = ctypes.byref(s)
    need = L.moe_workspace_size(_lib.MOE_OP_ROUTE, sh, _lib.MOE_BF16)
    planes = (3 * 16 * 64 * 2 + 255) // 256 * 256
    assert need == planes + (100 * 16 * 4 + 255) // 256 * 256
    assert _route(sh, ws=None) == -3
    assert _route(sh, wsb=planes - 1) == -3                           # the planes do not fit
    assert _route(sh, logits=None, wsb=need - 1) == -3                # nor the logits kept in ws
    assert _route(sh, ws=FAKE + 16) == -3                             # not 256-byte aligned
    # from given logits no workspace is used
    s0 = _sh(T=0)
    assert _route(ctypes.byref(s0), ws=None, wsb=0, flags=_lib.MOE_ROUTE_LOGITS_IN) == 0
    assert _route(ctypes.byref(s0), ws=FAKE, wsb=planes) == 0


def test_route_workspace_split_gate():
    """bf16 x with E = 256: with more than one split the partial products need
    the same workspace whether or not the caller keeps the logits; with one
    split (256 row tiles already fill the chip) the product writes the logits
    directly, so a caller that keeps them needs only the planes and the
    split's counters.  One byte less is rejected before anything is launched
    (fp32 x takes the plain product: planes, plus the logits only when they
    are not returned)."""
    planes = 3 * 256 * 512 * 2
    split = 768
    # (24 steps at d = 512: a split count divides them into even parts of at
    # least 4, so 6 at most)
    for T, S in ((1, 6), (300, 6), (16384, 4), (65536, 1)):
        s = _sh(T=T, d=512, E=256, G=8, M=4, k=8, gk=2)
        sh = ctypes.byref(s)
        need = L.moe_workspace_size(_lib.MOE_OP_ROUTE, sh, _lib.MOE_BF16)
        logits_bytes = (T * 256 * 4 + 255) // 256 * 256
        assert need == planes + split + (S if S > 1 else 1) * logits_bytes, (T, S)
        assert _route(sh, logits=None, wsb=need - 1) == -3, T
        kept = need if S > 1 else planes + split
        assert _route(sh, logits=FAKE, wsb=kept - 1) == -3, T
        need32 = L.moe_workspace_size(_lib.MOE_OP_ROUTE, sh, _lib.MOE_F32)
        assert need32 == planes + (T * 256 * 4 + 255) // 256 * 256
        assert _route(sh, xdt=_lib.MOE_F32, logits=None, wsb=need32 - 1) == -3
        assert _route(sh, xdt=_lib.MOE_F32, logits=FAKE, wsb=planes - 1) == -3


def test_route_workspace_split_small_gate():
    """bf16 x with E % 256 != 0 (E = 64, 64 x 64 tiles): the gate product is
    split over its 96 steps at d = 2048 until the launch reaches 256 tiles, so
    the workspace holds S partial products whether or not the caller keeps the
    logits (no split counters on this path); with one split the product writes
    the logits directly."""
    planes = 3 * 64 * 2048 * 2
    for T, S in ((77, 8), (4096, 4), (8192, 2), (16384, 1)):
        s = _sh(T=T, d=2048, E=64, G=8, M=4, k=6, gk=1)
        sh = ctypes.byref(s)
        need = L.moe_workspace_size(_lib.MOE_OP_ROUTE, sh, _lib.MOE_BF16)
        logits_bytes = (T * 64 * 4 + 255) // 256 * 256
        assert need == planes + (S if S > 1 else 1) * logits_bytes, (T, S)
        assert _route(sh, logits=None, wsb=need - 1) == -3, T
        kept = need if S > 1 else planes
        assert _route(sh, logits=FAKE, wsb=kept - 1) == -3, T


def test_route_unsupported_and_empty():
    sh = _sh(E=320, G=5, M=2, k=4, gk=2)
    assert _route(ctypes.byref(sh)) == -2
    sh0 = _sh(T=0)
    assert _route(ctypes.byref(sh0)) == 0


def test_workspace_sizes():
    ws = lambda op, s, dt=1: L.moe_workspace_size(op, ctypes.byref(s) if s is not None else None, dt)
    v3 = _lib.MoeShape(16384, 7168, 256, 8, 4, 8, 2, 2048)
    # dispatch: base rows per (64-token block, expert); e4m3 adds the scale table
    assert ws(_lib.MOE_OP_DISPATCH, v3, _lib.MOE_BF16) == 256 * 256 * 4
    assert ws(_lib.MOE_OP_DISPATCH, v3, _lib.MOE_E4M3) == 256 * 256 * 4 + 56 * 16384 * 4
    assert ws(_lib.MOE_OP_COMBINE, v3) == 0
    # expert products: two ticket-counter sets (9 counters on 64-byte lines each)
    assert ws(_lib.MOE_OP_EXPERT_FFN, v3) == 2 * 768
    assert ws(_lib.MOE_OP_EXPERT_FFN, None) == 2 * 768
    assert ws(_lib.MOE_OP_EXPERT_FFN_BACKWARD, v3) == 768
    # route: the weight planes; bf16 x at E = 256 splits the gate product in 4
    # over its 336 steps (64 row tiles x 4 = 256 tiles): its counters and
    # offsets (768 B), then 4 partial products; fp32 x: the logits
    assert ws(_lib.MOE_OP_ROUTE, v3) == 3 * 256 * 7168 * 2 + 768 + 4 * 16384 * 256 * 4
    assert ws(_lib.MOE_OP_ROUTE, v3, _lib.MOE_F32) == 3 * 256 * 7168 * 2 + 16384 * 256 * 4
    big = _lib.MoeShape(65536, 7168, 256, 8, 4, 8, 2, 2048)   # 256 row tiles: one split
    assert ws(_lib.MOE_OP_ROUTE, big) == 3 * 256 * 7168 * 2 + 768 + 65536 * 256 * 4
    assert ws(99, v3) == 0
    assert ws(_lib.MOE_OP_ROUTE, _lib.MoeShape(16, 64, 15, 4, 2, 4, 2, 32)) == 0   # invalid shape


def test_dispatch_checks():
    sh = _sh()
    ws = L.moe_workspace_size(_lib.MOE_OP_DISPATCH, ctypes.byref(sh), _lib.MOE_BF16)
    assert ws == 1 * 16 * 4
    args = lambda eb, ee, xdt, odt, scale, wsb: (ctypes.byref(sh), FAKE, FAKE, eb, ee, FAKE, xdt, odt, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, scale, FAKE, wsb, None)
    assert L.moe_dispatch(*args(0, 17, 1, 1, None, ws)) == -1
    assert L.moe_dispatch(*args(3, 3, 1, 1, None, ws)) == -1
    assert L.moe_dispatch(*args(0, 16, 1, 1, None, ws - 1)) == -3
    assert L.moe_dispatch(*args(0, 16, 1, 2, None, ws)) == -1          # e4m3 needs scales
    assert L.moe_dispatch(*args(0, 16, 0, 2, FAKE, ws)) == -2          # e4m3 from f32 x
    assert L.moe_dispatch(*args(0, 16, 1, 0, None, ws)) == -2          # bf16 -> f32 repack
    sh0 = _sh(T=0)
    assert L.moe_dispatch(ctypes.byref(sh0), FAKE, FAKE, 0, 16, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None, FAKE, 0, None) == 0


def test_expert_ffn_checks():
    W = L.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN, None, 1)
    f = lambda *a, ws=FAKE, wsb=W, ex=None: L.moe_expert_ffn(*a, ex, ws, wsb, None)
    assert f(0, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3) == -1
    assert f(2000, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3) == -1
    assert f(4, None, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3) == -1
    assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 0) == -1
    assert f(4, FAKE, 10, 64, 32, 1, None, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 1) == -1
    assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, None, None, FAKE, None, FAKE, 2) == -1
    assert f(4, FAKE, 10, 256, 128, 2, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3) == -1
    assert f(4, FAKE, 10, 200, 128, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3) == -2
    assert f(4, FAKE, 10, 512, 256, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, ws=None) == -3
    assert f(4, FAKE, 10, 512, 256, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, wsb=W - 1) == -3
    assert f(4, FAKE, 10, 512, 256, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3,
             ws=FAKE + 64) == -3
    assert f(4, FAKE, 0, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3) == 0
    # the extra group (shared expert): its buffers are checked like the routed ones
    good = dict(rows=16, x=FAKE, w13=FAKE, w2=FAKE, h=FAKE, y=FAKE)
    ex = lambda **kw: ctypes.byref(_lib.MoeFfnExtra(**{**good, **kw}))
    assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3,
             ex=ex(rows=-1)) == -1
    for k in ("x", "w13", "w2", "h", "y"):
        assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3,
                 ex=ex(**{k: None})) == -1, k
    # e4m3 needs the extra group's scales too
    assert f(4, FAKE, 10, 256, 128, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3,
             ex=ex()) == -1
    # rows = 0 is no extra group: an empty call stays a no-op
    assert f(4, FAKE, 0, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3,
             ex=ex(rows=0)) == 0


def test_combine_checks():
    sh = _sh()
    c = L.moe_combine
    assert c(ctypes.byref(sh), None, FAKE, FAKE, 1, None, FAKE, 1, 0, None) == -1
    assert c(ctypes.byref(sh), FAKE, FAKE, FAKE, 2, None, FAKE, 1, 0, None) == -1
    assert c(ctypes.byref(sh), FAKE, FAKE, FAKE, 1, None, FAKE, 1, 1, None) == -2   # += needs f32 out
    assert c(ctypes.byref(sh), FAKE, FAKE, FAKE, 1, None, FAKE, 0, 2, None) == -1
    sh0 = _sh(T=0)
    assert c(ctypes.byref(sh0), FAKE, FAKE, FAKE, 1, None, FAKE, 1, 0, None) == 0


def test_prep_checks():
    assert L.moe_quantize_blocks_e4m3(1, 100, 128, FAKE, FAKE, FAKE, None) == -2
    assert L.moe_quantize_blocks_e4m3(1, 128, 128, None, FAKE, FAKE, None) == -1
    assert L.moe_quantize_blocks_e4m3(0, 128, 128, FAKE, FAKE, FAKE, None) == 0


def test_bias_update_checks():
    bad = ctypes.c_void_p(16)  # never dereferenced: every case below fails on the host
    assert L.moe_bias_update(0, 16, None, 0.01, None, None, None) == _lib.MOE_OK  # no rows: no-op
    assert L.moe_bias_update(-1, 16, bad, 0.01, bad, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(4, 0, bad, 0.01, bad, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(4, 1025, bad, 0.01, bad, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(4, 16, None, 0.01, bad, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_bias_update(4, 16, bad, 0.01, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    for g in (float("inf"), float("nan")):
        assert L.moe_bias_update(4, 16, bad, g, bad, None, None) == _lib.MOE_ERR_INVALID_ARG


def test_route_hash_checks():
    bad = ctypes.c_void_p(16)  # never dereferenced: every case below fails on the host
    def sh(T, E, k):
        return ctypes.byref(_lib.MoeShape(T, 64, E, 1, 1, k, 1, 32))
    assert L.moe_route_hash(sh(0, 16, 4), None, 1, None, None, None, None, None) == _lib.MOE_OK
    assert L.moe_route_hash(None, bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_hash(sh(-1, 16, 4), bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_hash(sh(8, 4, 5), bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_hash(sh(8, 16, 0), bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_hash(sh(8, 2048, 4), bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_route_hash(sh(8, 64, 17), bad, 1, None, bad, bad, bad, None) == _lib.MOE_ERR_UNSUPPORTED
    for i in range(4):
        ptrs = [bad, bad, bad, bad]
        ptrs[i] = None
        assert L.moe_route_hash(sh(8, 16, 4), ptrs[0], 1, None, ptrs[1], ptrs[2], ptrs[3],
                                None) == _lib.MOE_ERR_INVALID_ARG


def test_backward_checks():
    bad = ctypes.c_void_p(16)  # never dereferenced: every case below fails on the host
    sh = lambda T=8, d=256, E=16, k=4: ctypes.byref(_lib.MoeShape(T, d, E, 4, 2, k, 2, 256))
    BF, F = _lib.MOE_BF16, _lib.MOE_F32
    # combine backward
    assert L.moe_combine_backward(sh(0), None, None, None, BF, None, BF, None, None, None) == _lib.MOE_OK
    assert L.moe_combine_backward(None, bad, bad, bad, BF, bad, BF, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_combine_backward(sh(), bad, bad, bad, 7, bad, BF, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_combine_backward(sh(k=17), bad, bad, bad, BF, bad, BF, bad, bad, None) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_combine_backward(sh(), None, bad, bad, BF, bad, BF, bad, bad, None) == _lib.MOE_ERR_INVALID_ARG
    # expert FFN backward
    WB = L.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN_BACKWARD, None, BF)
    fb = lambda *a, ws=FAKE, wsb=WB: L.moe_expert_ffn_backward(*a, ws, wsb, None)
    args = [bad] * 10
    assert fb(0, bad, 8, 256, 256, BF, *args, 0) == _lib.MOE_ERR_INVALID_ARG
    assert fb(2, None, 8, 256, 256, BF, *args, 0) == _lib.MOE_ERR_INVALID_ARG
    assert fb(1, None, 8, 256, 256, BF, *args, 2) == _lib.MOE_ERR_INVALID_ARG
    assert fb(1, None, 8, 256, 256, F, *args, 0) == _lib.MOE_ERR_UNSUPPORTED
    assert fb(1, None, 8, 256, 128, BF, *args, 0) == _lib.MOE_ERR_UNSUPPORTED
    assert fb(1, None, 8, 200, 256, BF, *args, 0) == _lib.MOE_ERR_UNSUPPORTED
    assert fb(1, None, 8, 256, 256, BF, *args, 0, ws=None) == _lib.MOE_ERR_WORKSPACE
    assert fb(1, None, 8, 256, 256, BF, *args, 0, wsb=WB - 1) == _lib.MOE_ERR_WORKSPACE
    for i in range(10):
        a = list(args)
        a[i] = None
        assert fb(1, None, 8, 256, 256, BF, *a, 0) == _lib.MOE_ERR_INVALID_ARG
    # training forward
    WT = L.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN, None, BF)
    ft = lambda *a, ws=FAKE, wsb=WT: L.moe_expert_ffn_train(*a, ws, wsb, None)
    targs = [bad] * 6
    assert ft(1, None, 0, 256, 256, BF, *targs) == _lib.MOE_OK
    assert ft(2, None, 8, 256, 256, BF, *targs) == _lib.MOE_ERR_INVALID_ARG
    assert ft(1, None, 8, 256, 128, BF, *targs) == _lib.MOE_ERR_UNSUPPORTED
    assert ft(1, None, 8, 256, 256, F, *targs) == _lib.MOE_ERR_UNSUPPORTED
    assert ft(1, None, 8, 256, 256, BF, *targs, wsb=WT - 1) == _lib.MOE_ERR_WORKSPACE
    for i in range(6):
        a = list(targs)
        a[i] = None
        assert ft(1, None, 8, 256, 256, BF, *a) == _lib.MOE_ERR_INVALID_ARG
    # dispatch backward
    assert L.moe_dispatch_backward(sh(0), None, None, BF, None, None, 0, None) == _lib.MOE_OK
    assert L.moe_dispatch_backward(sh(), bad, bad, BF, None, bad, 2, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_backward(sh(), None, bad, BF, None, bad, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_backward(sh(d=12), bad, bad, BF, None, bad, 0, None) == _lib.MOE_ERR_UNSUPPORTED
    # route backward
    assert L.moe_route_backward(sh(0), None, BF, None, None, None, None, None, None, None, None,
                                None, 0, None) == _lib.MOE_OK
    assert L.moe_route_backward(sh(k=20), bad, BF, bad, None, bad, bad, bad, bad, bad, bad,
                                None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_backward(sh(), bad, 9, bad, None, bad, bad, bad, bad, bad, bad,
                                None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_backward(sh(), bad, BF, None, None, bad, bad, bad, bad, bad, bad,
                                None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    big = ctypes.byref(_lib.MoeShape(16384, 7168, 256, 8, 4, 8, 2, 2048))
    need = L.moe_workspace_size(_lib.MOE_OP_ROUTE_BACKWARD, big, BF)
    # the larger of the two paths: 16 fp32 K-parts of dW_g, or the bf16-plane
    # path (dlogits as 6 and 3 planes, W_g as 6 planes, 8 row splits of fp32
    # [d, 3E] partials, one ticket-counter set)
    T, d, E = 16384, 7168, 256
    assert need == max(16 * d * E * 4,
                       T * 6 * E * 2 + d * 6 * E * 2 + T * 3 * E * 2 + 8 * d * 3 * E * 4 + 9 * 64)
    assert L.moe_route_backward(big, bad, BF, bad, None, bad, bad, bad, bad, bad, bad, FAKE, need - 1,
                                None) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE_BACKWARD, sh(T=1000), BF) == 0


def test_dispatch_noalloc_host_checks():
    """Argument and size checks on the host, before the static scratch (or
    anything on a device) is touched."""
    f = L.moe_dispatch_noalloc
    big = _lib.MoeShape(65536, 7168, 256, 8, 4, 8, 2, 2048)
    # e4m3 output: 56 x 65536 fp32 scales alone exceed the 8 MiB scratch
    assert f(ctypes.byref(big), FAKE, FAKE, 0, 256, FAKE, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
             None) == _lib.MOE_ERR_SCRATCH
    assert _lib.MOE_DISPATCH_NOALLOC_SCRATCH == 8 << 20
    need = L.moe_workspace_size(_lib.MOE_OP_DISPATCH, ctypes.byref(big), _lib.MOE_E4M3)
    assert need > _lib.MOE_DISPATCH_NOALLOC_SCRATCH
    sh = _sh()
    assert f(ctypes.byref(sh), None, FAKE, 0, 16, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
             None) == _lib.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), FAKE, FAKE, 0, 17, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
             None) == _lib.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(sh), FAKE, FAKE, 0, 16, FAKE, 1, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None,
             None) == _lib.MOE_ERR_INVALID_ARG          # e4m3 needs scales
    sh0 = _sh(T=0)
    assert f(ctypes.byref(sh0), FAKE, FAKE, 0, 16, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
             None) == _lib.MOE_OK
