"""Pins for the oracle's e4m3 quantisation against torch's float8_e4m3fn cast
(a library routine) and against the format's definition."""
import numpy as np
import torch

from oracle import fp8 as Q


def _torch_codes(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_dense_sweep():
    top = np.float32(448.0).view(np.uint32)
    pos = np.arange(0, top + 1, 7, dtype=np.uint32).view(np.float32)
    v = np.concatenate([pos, -pos])
    assert np.array_equal(Q.to_e4m3(v), _torch_codes(v))


def test_matches_torch_on_midpoints():
    t = Q.e4m3_table()
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    v = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)]).astype(np.float32)
    assert np.array_equal(Q.to_e4m3(v), _torch_codes(v))


def test_cast_equals_definition():
    # the library cast the quantisers round through gives the definition's codes
    t = Q.e4m3_table()
    mids = ((t[1:] + t[:-1]) / 2).astype(np.float32)
    top = np.float32(448.0).view(np.uint32)
    sweep = np.arange(0, top + 1, 13, dtype=np.uint32).view(np.float32)
    sat = np.array([448.0, 448.00003, 463.9, 464.0, 479.9, 480.0, 1e6, 3.4e38, -0.0, 1e-30, -1e-30],
                   dtype=np.float32)
    v = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1000), sweep, sat])
    v = np.concatenate([v, -v])
    assert np.array_equal(Q.to_e4m3_cast(v), Q.to_e4m3(v))


def test_quantisers_same_with_either_rounding():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((37, 512)) * np.exp(rng.uniform(-8, 8, size=(37, 1)))).astype(np.float32)
    x[3, :128] = 0.0
    a, sa = Q.quantize_rows(x)
    b, sb = Q.quantize_rows(x, cast=Q.to_e4m3)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
    w = (0.02 * rng.standard_normal((256, 384))).astype(np.float32)
    w[:128, 128:256] = 0.0
    a, sa = Q.quantize_blocks(w)
    b, sb = Q.quantize_blocks(w, cast=Q.to_e4m3)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_round_trip_and_format():
    t = Q.e4m3_table()
    assert t[-1] == 448.0 and t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(Q.to_e4m3(Q.from_e4m3(codes)), codes)
    assert np.array_equal(Q.to_e4m3(-Q.from_e4m3(codes[1:])), codes[1:] | 0x80)


def test_saturation_and_relative_error():
    assert Q.to_e4m3(np.float32(1e6)) == 0x7E and Q.to_e4m3(np.float32(-500.0)) == 0xFE
    v = np.geomspace(2.0 ** -6, 448, 100000).astype(np.float32)
    r = Q.from_e4m3(Q.to_e4m3(v)).astype(np.float64)
    assert np.all(np.abs(r - v) <= 2.0 ** -4 * np.abs(v))


def test_tile_quantisation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[2, :128] = 0.0
    q, s = Q.quantize_rows(x)
    assert s.shape == (6, 2) and s[2, 0] == 1.0
    amax = np.abs(x.reshape(6, 2, 128)).max(2)
    ok = amax > 0
    assert np.array_equal(s[ok], (amax[ok] / np.float32(448)).astype(np.float32))
    # the element of largest magnitude lands on +-448 (or one step below)
    deq = Q.dequant_rows(q, s)
    assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -9 * s.repeat(128, 1))
    w = (0.02 * rng.standard_normal((256, 384))).astype(np.float32)
    qw, sw = Q.quantize_blocks(w)
    assert sw.shape == (2, 3)
    assert np.abs(Q.dequant_blocks(qw, sw) - w).max() <= 2.0 ** -4 * np.abs(w).max()
