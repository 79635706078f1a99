"""Pins of the oracle's OCP E4M3 codec and row quantiser (CPU only).

The codec is checked against torch's float8_e4m3fn conversions (an
independent library implementation of the same OCP format), against values
the format definition fixes, and against its rounding rule on exact ties.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as F8


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def test_decode_matches_library_for_every_code():
    ref = _torch_decode_all()
    got = F8.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_values_fixed_by_the_format():
    d = F8.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5
    assert d(0x00) == 0.0 and np.signbit(d(0x80))


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(F8.e4m3_encode(F8.e4m3_decode(codes)), codes.astype(np.uint8))


def test_encode_matches_library_rounding():
    g = np.random.default_rng(7)
    mags = np.exp2(g.uniform(-12, np.log2(448.0), size=20000))
    v = (mags * g.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F8.e4m3_encode(v.astype(np.float64)), ref)


def test_encode_ties_go_to_the_even_code():
    # midpoints between neighbouring finite magnitudes: the code with an even
    # mantissa (low bit 0) wins
    vals = F8.e4m3_decode(np.arange(0x00, 0x7F))
    mids = (vals[:-1] + vals[1:]) / 2.0
    got = F8.e4m3_encode(mids).astype(np.int64)
    lo = np.arange(0x00, 0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)


def test_encode_saturates():
    assert list(F8.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_quantize_rows_scale_bound_and_zero_row():
    g = np.random.default_rng(3)
    w = g.normal(0, 0.02, size=(64, 300)).astype(np.float32)
    w[5] = 0.0
    w[6, :] = 0.0
    w[6, 17] = -3.0e-5
    q, s = F8.quantize_rows(w)
    assert s.dtype == np.float32
    # the scale is the fp32 quotient amax / 448 (library fp32 division)
    amax = torch.from_numpy(np.abs(w)).amax(dim=1)
    want = torch.where(amax > 0, amax / torch.tensor(448.0), torch.tensor(1.0)).numpy()
    assert np.array_equal(s, want)
    assert s[5] == 1.0 and not q[5].any()
    nz = np.abs(w).max(axis=1) > 0
    assert ((q[nz] & 0x7F).max(axis=1) == 0x7E).all()      # the row maximum maps to 448
    # reconstruction error is at most half a step of the format at that magnitude
    deq = F8.dequantize_rows(q, s)
    r = np.abs(w.astype(np.float64) / s[:, None].astype(np.float64))
    step = np.where(r < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(r, 2.0 ** -6))) - 3))
    err = np.abs(deq - w) / s[:, None]
    assert (err <= step / 2 * (1 + 1e-6) + 1e-12).all()
    assert deq[6, 17] == -float(s[6]) * 448.0


def test_quantize_experts_shapes():
    w = {n: np.random.default_rng(1).normal(0, 0.02, size=sh).astype(np.float32)
         for n, sh in (("w_gate", (3, 8, 16)), ("w_up", (3, 8, 16)), ("w_down", (3, 16, 8)),
                       ("ws_gate", (8, 16)), ("ws_up", (8, 16)), ("ws_down", (16, 8)))}
    codes, scales, deq = F8.quantize_experts(w)
    assert codes["w_gate"].shape == (3, 8, 16) and scales["w_gate"].shape == (3, 8)
    assert scales["ws_down"].shape == (16,)
    q, s = F8.quantize_rows(w["w_down"][2])
    assert np.array_equal(codes["w_down"][2], q) and np.array_equal(scales["w_down"][2], s)
    assert np.allclose(deq["w_up"], w["w_up"], atol=0.02 * 4 / 448 * 16)
