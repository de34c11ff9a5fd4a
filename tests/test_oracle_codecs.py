"""Pins for the oracle's BF16/FP8 decoders and encoders.

Each check ties the oracle to something other than itself: values printed on
the pages (tests/golden), torch's independent float8/bfloat16 casts, a
brute-force nearest-code search, or structural facts of the formats.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}
TORCH_FP8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def all_codes():
    return np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_fp8_max_and_fields_match_pages(name):
    g = json.load(open(os.path.join(GOLDEN, "fp8_formats.json")))[name]
    vals = oracle.decode_fp8(all_codes(), FMT[name])
    finite = vals[np.isfinite(vals)]
    assert finite.max() == g["max_normal"]
    assert finite.min() == -g["max_normal"]
    assert np.isinf(vals).any() == g["has_inf"]
    # mantissa bits: every binade of normals holds 2^mantissa evenly spaced values
    mb, eb = g["mantissa"], g["exponent"]
    pos = np.unique(finite[finite > 0])
    one_binade = pos[(pos >= 1.0) & (pos < 2.0)]
    assert len(one_binade) == 2 ** mb
    assert np.allclose(np.diff(one_binade), 2.0 ** -mb)
    # exponent bits: bias 2^(eb-1)-1 puts the smallest normal at 2^(1-bias)
    bias = 2 ** (eb - 1) - 1
    assert np.min(pos[pos >= 2.0 ** (1 - bias)]) == 2.0 ** (1 - bias)
    # subnormal step = 2^(1-bias-mb)
    assert pos.min() == 2.0 ** (1 - bias - mb)


def test_bf16_fields_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "fp8_formats.json")))["bf16"]
    codes = np.arange(65536, dtype=np.uint16)
    vals = oracle.decode_bf16(codes)
    pos = np.unique(vals[np.isfinite(vals) & (vals > 0)])
    assert len(pos[(pos >= 1.0) & (pos < 2.0)]) == 2 ** g["mantissa"]
    # same exponent range as FP32
    assert pos.max() == (2 - 2.0 ** -7) * 2.0 ** 127
    assert pos.min() == 2.0 ** -133


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp8_decode_matches_torch(fmt):
    codes = all_codes()
    ours = oracle.decode_fp8(codes, fmt)
    ref = torch.from_numpy(codes).view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    # sign symmetry and strict monotonicity over positive finite codes
    assert np.array_equal(ours[128:][m[:128]], -ours[:128][m[:128]])
    posfin = ours[:128][np.isfinite(ours[:128])]
    assert np.all(np.diff(posfin) > 0)


def test_bf16_decode_matches_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oracle.decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])


def test_fp8_encode_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "fp8_encode_cases.json")))["cases"]
    for name, x, code, why in cases:
        got = int(oracle.encode_fp8(np.array([x], np.float32), FMT[name])[0])
        assert got == code, (name, x, code, got, why)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp8_encode_roundtrip_all_codes(fmt):
    codes = all_codes()
    vals = oracle.decode_fp8(codes, fmt)
    fin = np.isfinite(vals)
    back = oracle.encode_fp8(vals[fin].astype(np.float32), fmt)
    assert np.array_equal(back, codes[fin])
    assert oracle.encode_fp8(np.array([np.nan, -np.nan], np.float32), fmt)[0] == 0x7F


def brute_force_fp8(x, fmt):
    """Nearest finite code by exhaustive search over the codomain, ties to the
    even code, with saturation at +-max (independent of the oracle's
    exponent/quantum arithmetic)."""
    codes = np.arange(128, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    keep = np.isfinite(vals)
    codes, vals = codes[keep], vals[keep]
    fmax = vals.max()
    x = np.asarray(x, np.float64).ravel()
    out = np.empty(x.shape, np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    for s in range(0, x.size, 65536):
        aa = a[s:s + 65536]
        d = np.abs(aa[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        tie = d == dmin
        # among the nearest codes (one or two), prefer the even one
        pick = np.where(tie & (codes[None, :] % 2 == 0), 1, 0) + tie
        idx = np.argmax(pick, axis=1)
        c = codes[idx]
        c = np.where(aa >= fmax, codes[np.argmax(vals)], c)
        out[s:s + 65536] = c
    out |= sign
    return out


def fp8_probe_values(fmt, rng):
    codes = np.arange(128, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    vals = np.unique(vals[np.isfinite(vals)])
    mids = (vals[:-1] + vals[1:]) / 2
    f32 = np.concatenate([vals, mids, vals[-1:] * 1.03, vals[-1:] * 1.1]).astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf))
    dn = np.nextafter(f32, np.float32(0))
    rnd = (rng.standard_normal(200000) * 2.0 ** rng.integers(-20, 18, 200000)).astype(np.float32)
    x = np.concatenate([f32, up, dn, rnd])
    return np.concatenate([x, -x])


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp8_encode_matches_brute_force(fmt):
    x = fp8_probe_values(fmt, np.random.default_rng(11))
    assert np.array_equal(oracle.encode_fp8(x, fmt), brute_force_fp8(x, fmt))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp8_encode_matches_torch_in_range(fmt):
    # torch's cast rounds to nearest even but does not saturate; compare where
    # no saturation happens.
    x = fp8_probe_values(fmt, np.random.default_rng(12))
    x = x[np.abs(x) < oracle.FMAX[fmt]]
    ref = torch.from_numpy(x).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8(x, fmt), ref)


def bf16_probe_patterns(rng):
    hi = np.arange(65536, dtype=np.uint32) << 16
    mids = hi | 0x8000
    pats = np.concatenate([hi, mids, mids + 1, mids - 1, hi | 0x7FFF, hi | 0x0001,
                           rng.integers(0, 2 ** 32, 2 ** 21, dtype=np.uint64).astype(np.uint32)])
    return pats.view(np.float32)


def test_bf16_encode_matches_torch():
    x = bf16_probe_patterns(np.random.default_rng(13))
    ours = oracle.encode_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN keeps its sign and becomes the quiet NaN 0x7FC0
    assert np.all((ours[nan] & 0x7FFF) == 0x7FC0)
    assert np.array_equal(ours[nan] >> 15, (x[nan].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_encode_matches_nearest_neighbour():
    # brute force: compare the two BF16 neighbours of x in FP64
    rng = np.random.default_rng(14)
    x = bf16_probe_patterns(rng)
    x = x[np.isfinite(x)][::7]
    u = x.view(np.uint32)
    lo = (u & 0xFFFF0000).view(np.float32).astype(np.float64)       # truncation toward 0
    hi_bits = (u & 0xFFFF0000) + 0x10000
    hi = hi_bits.view(np.float32).astype(np.float64)                   # next code away from 0
    # IEEE overflow rule: round as if the exponent were unbounded; the code
    # after the largest finite one then stands for 2^128 and means Inf
    xd = x.astype(np.float64)
    hi = np.where(np.isinf(hi), np.copysign(2.0 ** 128, xd), hi)
    dlo, dhi = np.abs(xd - lo), np.abs(hi - xd)
    lo_code = (u >> 16).astype(np.uint16)
    hi_code = (hi_bits >> 16).astype(np.uint16)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo_code % 2 == 1))
    expect = np.where(pick_hi, hi_code, lo_code)
    assert np.array_equal(oracle.encode_bf16(x), expect)
