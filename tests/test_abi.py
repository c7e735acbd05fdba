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
    st = L.moe_route(ctypes.byref(sh), FAKE, _lib.MOE_BF16, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None)
    assert st == _lib.MOE_ERR_INVALID_ARG


def test_route_rejects_null_and_flags():
    sh = _sh()
    assert L.moe_route(None, FAKE, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == -1
    assert L.moe_route(ctypes.byref(sh), FAKE, 1, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 0, None) == -1
    assert L.moe_route(ctypes.byref(sh), None, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == -1
    assert L.moe_route(ctypes.byref(sh), FAKE, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, None) == -1
    assert L.moe_route(ctypes.byref(sh), FAKE, 7, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == -1


def test_route_unsupported_and_empty():
    sh = _sh(E=320, G=5, M=2, k=4, gk=2)
    assert L.moe_route(ctypes.byref(sh), FAKE, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == -2
    sh0 = _sh(T=0)
    assert L.moe_route(ctypes.byref(sh0), FAKE, 1, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == 0


def test_dispatch_checks():
    sh = _sh()
    ws = L.moe_dispatch_workspace_size(ctypes.byref(sh), 0, 16)
    assert ws == 1 * 16 * 4
    assert L.moe_dispatch_workspace_size(ctypes.byref(sh), 4, 2) == 0
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
    f = L.moe_expert_ffn
    assert f(0, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, None) == -1
    assert f(2000, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, None) == -1
    assert f(4, None, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, None) == -1
    assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 0, None) == -1
    assert f(4, FAKE, 10, 64, 32, 1, None, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 1, None) == -1
    assert f(4, FAKE, 10, 64, 32, 1, FAKE, None, FAKE, None, None, None, FAKE, None, FAKE, 2, None) == -1
    assert f(4, FAKE, 10, 256, 128, 2, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, None) == -1
    assert f(4, FAKE, 10, 200, 128, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, None) == -2
    assert f(4, FAKE, 0, 64, 32, 1, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 3, None) == 0


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
    assert L.moe_gate_prepare(0, 16, FAKE, FAKE, None) == -1
    assert L.moe_gate_prepare(64, 16, None, FAKE, None) == -1
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
    args = [bad] * 10
    assert L.moe_expert_ffn_backward(0, bad, 8, 256, 256, BF, *args, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_backward(2, None, 8, 256, 256, BF, *args, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_backward(1, None, 8, 256, 256, BF, *args, 2, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_backward(1, None, 8, 256, 256, F, *args, 0, None) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_ffn_backward(1, None, 8, 256, 128, BF, *args, 0, None) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_ffn_backward(1, None, 8, 200, 256, BF, *args, 0, None) == _lib.MOE_ERR_UNSUPPORTED
    for i in range(10):
        a = list(args)
        a[i] = None
        assert L.moe_expert_ffn_backward(1, None, 8, 256, 256, BF, *a, 0, None) == _lib.MOE_ERR_INVALID_ARG
    # training forward
    targs = [bad] * 6
    assert L.moe_expert_ffn_train(1, None, 0, 256, 256, BF, *targs, None) == _lib.MOE_OK
    assert L.moe_expert_ffn_train(2, None, 8, 256, 256, BF, *targs, None) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn_train(1, None, 8, 256, 128, BF, *targs, None) == _lib.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_ffn_train(1, None, 8, 256, 256, F, *targs, None) == _lib.MOE_ERR_UNSUPPORTED
    for i in range(6):
        a = list(targs)
        a[i] = None
        assert L.moe_expert_ffn_train(1, None, 8, 256, 256, BF, *a, None) == _lib.MOE_ERR_INVALID_ARG
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
    need = L.moe_route_backward_workspace_size(big)
    # the larger of the two paths: 16 fp32 K-parts of dW_g, or the bf16-plane
    # path (dlogits as 6 and 3 planes, W_g as 6 planes, 8 row splits of fp32
    # [d, 3E] partials)
    T, d, E = 16384, 7168, 256
    assert need == max(16 * d * E * 4, T * 6 * E * 2 + d * 6 * E * 2 + T * 3 * E * 2 + 8 * d * 3 * E * 4)
    assert L.moe_route_backward(big, bad, BF, bad, None, bad, bad, bad, bad, bad, bad, bad, need - 1,
                                None) == _lib.MOE_ERR_WORKSPACE
    assert L.moe_route_backward_workspace_size(sh(T=1000)) == 0
