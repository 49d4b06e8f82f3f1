"""Pins of the oracle's number codecs against the format definitions and torch's casts.

The FP8 format is OCP E4M3FN (one reading of the pages, which say only "FP8");
bf16 is the upper half of binary32 with round-to-nearest-even.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_to_f32(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def _torch_f32_to_e4m3(v):
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = _torch_e4m3_to_f32(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_special_values_from_format_definition(oracle):
    with open(os.path.join(GOLD, "e4m3_special_values.json")) as f:
        gold = json.load(f)
    for item in gold["values"]:
        code = int(item["code"], 16)
        assert oracle.e4m3_decode([code])[0] == float(item["value"]), item


def _nonneg_finite_values(oracle):
    return oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def test_e4m3_encode_midpoints_and_neighbours_match_torch(oracle):
    vals = _nonneg_finite_values(oracle)
    mids = (vals[:-1] + vals[1:]) / 2
    f32 = mids.astype(np.float32)
    probes = np.concatenate([vals, f32, np.nextafter(f32, np.float32(1e9)), np.nextafter(f32, np.float32(-1e9))])
    probes = np.concatenate([probes, -probes]).astype(np.float32)
    ours = oracle.e4m3_encode(probes.astype(np.float64))
    ref = _torch_f32_to_e4m3(probes)
    # -0.0 encodes to 0x80 in both; compare bitwise
    assert np.array_equal(ours, ref)


def test_e4m3_encode_random_match_torch(oracle):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(5000) * 1e-3]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), _torch_f32_to_e4m3(v))


def test_e4m3_encode_saturates_and_nan(oracle):
    # our rule: finite magnitudes >= 448 saturate to +-448; NaN -> 0x7F
    assert oracle.e4m3_encode([448.0, 449.0, 1e30, -500.0]).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.e4m3_encode([float("nan")]).tolist() == [0x7F]


def test_e4m3_encode_is_nearest_code_brute_force(oracle):
    """Brute force over all 253 finite codes: the chosen code is at minimal distance."""
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = ~np.isnan(vals)
    rng = np.random.default_rng(11)
    for v in rng.uniform(-448, 448, 3000):
        c = int(oracle.e4m3_encode([v])[0])
        d = np.abs(vals[finite] - v).min()
        assert abs(vals[c] - v) == d


def test_bf16_encode_random_bits_match_torch(oracle):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_encode(f), ref)


def test_bf16_encode_ties_to_even(oracle):
    # 1 + 2^-8 is exactly half-way between bf16 1.0 and 1.0078125: even -> 1.0
    assert oracle.bf16_encode([1.0 + 2**-8]).tolist() == [0x3F80]
    # 1.0078125 + 2^-8 is half-way between 0x3F81 and 0x3F82: even -> 0x3F82
    assert oracle.bf16_encode([1.0078125 + 2**-8]).tolist() == [0x3F82]
    assert oracle.bf16_decode([0x3F80, 0xBF80, 0x4049]).tolist() == [1.0, -1.0, 3.140625]


def test_requant_chunk_matches_torch_pipeline(oracle):
    """FP8 requantisation of the intermediate: s = amax/448, cast, multiply back."""
    rng = np.random.default_rng(8)
    for scale in (1e-3, 1.0, 30.0):
        a = (rng.standard_normal(128) * scale).astype(np.float32)
        s = np.float32(np.abs(a).max() / np.float32(448.0))
        q = _torch_e4m3_to_f32(_torch_f32_to_e4m3((a / s).astype(np.float32)))
        ref = (q.astype(np.float32) * s).astype(np.float32)
        got = oracle.requant_chunk(a)
        assert np.array_equal(got.astype(np.float32), ref)
        # the largest element maps to +-448 * s exactly
        i = int(np.argmax(np.abs(a)))
        assert abs(got[i]) == np.float32(448.0) * s


def test_requant_chunk_all_zero(oracle):
    assert np.array_equal(oracle.requant_chunk(np.zeros(128)), np.zeros(128))


# ----------------------------------------------------------------- MXFP8
def test_e8m0_decode_all_bytes(oracle):
    """E8M0 byte s is the biased exponent of 2^(s-127) (the binary32 with exponent
    field s and zero mantissa for s in 1..254; s = 0 is 2^-127, s = 255 is NaN)."""
    s = np.arange(256, dtype=np.uint32)
    got = oracle.e8m0_decode(s.astype(np.uint8))
    ref = (s[1:255] << 23).view(np.float32).astype(np.float64)
    assert np.array_equal(got[1:255], ref)
    assert got[0] == 2.0 ** -127 and np.isnan(got[255])


def _torch_mx_block(v):
    """MX quantise-dequantise of one block, from the format's definition, by torch:
    X = floor(log2(amax)) - 8; e4m3 cast of v / 2^X clamped to +-448; times 2^X."""
    import torch
    t = torch.tensor(v, dtype=torch.float64)
    amax = float(t.abs().max())
    if amax == 0:
        return t.numpy(), 127
    x = math.floor(math.log2(amax)) - 8
    q = torch.clamp(t / 2.0 ** x, -448, 448).float().to(torch.float8_e4m3fn).double()
    return (q * 2.0 ** x).numpy(), x + 127


def test_mx_requant_block_matches_definition(oracle):
    rng = np.random.default_rng(4)
    cases = [rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6) for _ in range(200)]
    cases += [np.zeros(32), np.full(32, 2.0 ** 5), np.linspace(-1, 1, 32) * 1.9 * 2.0 ** 3,
              np.r_[448.0 * 2 ** -8, np.zeros(31)], rng.standard_normal(32) * 1e-30]
    for v in cases:
        got, b = oracle.mx_requant_block(v)
        ref, rb = _torch_mx_block(v)
        assert b == rb
        assert np.array_equal(got, ref)


def test_mx_requant_saturates_and_brackets_amax(oracle):
    """The shared exponent puts amax in [2^(X+8), 2^(X+9)); quotients above 448 clamp."""
    v = np.zeros(32)
    v[0] = 1.99 * 2 ** 4   # amax: X = 4 - 8 = -4, quotient 1.99 * 2^8 = 509.4 -> 448
    v[1] = -0.75
    got, b = oracle.mx_requant_block(v)
    assert b == 127 - 4
    assert got[0] == 448.0 * 2.0 ** -4 and got[1] == -0.75
    for _ in range(50):
        w = np.random.default_rng(_).standard_normal(32) * 3.0
        _, b = oracle.mx_requant_block(w)
        amax = np.abs(w).max()
        assert 2.0 ** (b - 127 + 8) <= amax < 2.0 ** (b - 127 + 9)
