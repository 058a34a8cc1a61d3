"""Pins for the oracle's element codecs (CPU only).

bf16 widening and OCP E4M3 decoding are checked code by code against torch's
own dtype conversions (library routines); E4M3 encoding against torch's
float -> float8_e4m3fn conversion (round-to-nearest-even) inside the finite
range, against an independent nearest-value search written here, and against
the saturation rule outside it; the fp32 division against numpy's IEEE
float32 division.
"""
import numpy as np
import pytest
import torch

import oracle


def test_bf16_widening_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _torch_e4m3_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes():
    ref = _torch_e4m3_decode()
    got = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    assert np.isnan(ref[0x7F]) and np.isnan(ref[0xFF])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # the format's landmarks: largest finite, smallest subnormal, one
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert got[0x80] == 0.0 and np.signbit(got[0x80])


def _nearest_even_encode(x: float) -> int:
    """Independent encoder: nearest finite E4M3 magnitude, ties to the code
    with an even mantissa, saturating at 448."""
    mags = np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)])  # 0x00..0x7E
    a = abs(float(x))
    sign = 0x80 if np.signbit(x) else 0
    if a >= 448.0:
        return sign | 0x7E
    diff = np.abs(mags - a)
    best = np.flatnonzero(diff == diff.min())
    code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
    return sign | code


def test_e4m3_encode_all_bf16_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    finite = torch.isfinite(vals) & (vals.abs() <= 448.0)
    ref = vals[finite].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_from_f32(v) for v in vals[finite].numpy()], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturation_and_nan():
    for v, code in [(448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E),
                    (float("inf"), 0x7E), (-500.0, 0xFE), (float("-inf"), 0xFE)]:
        assert oracle.e4m3_from_f32(v) == code, v
    assert oracle.e4m3_from_f32(float("nan")) & 0x7F == 0x7F
    assert oracle.e4m3_from_f32(0.0) == 0x00 and oracle.e4m3_from_f32(-0.0) == 0x80
    # ties: 2^-10 is halfway between 0 and the smallest subnormal -> even (0)
    assert oracle.e4m3_from_f32(2.0 ** -10) == 0x00
    assert oracle.e4m3_from_f32(3 * 2.0 ** -10) == 0x02  # 1.5 ulp -> 2 (even)
    assert oracle.e4m3_from_f32(1.0 + 1 / 16) == 0x38     # tie between 1 and 1.125 -> 1
    assert oracle.e4m3_from_f32(1.0 + 3 / 16) == 0x3A     # tie between 1.125 and 1.25 -> 1.25


def test_e4m3_encode_vs_nearest_search():
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.standard_normal(1500).astype(np.float32) * 40,
        (rng.standard_normal(500) * 1e-2).astype(np.float32),
        np.float32([oracle.e4m3_to_f64(c) for c in range(0x7F)]),
        # exact midpoints between neighbouring codes
        np.float32([(oracle.e4m3_to_f64(c) + oracle.e4m3_to_f64(c + 1)) / 2 for c in range(0x7E)]),
    ])
    for x in xs:
        assert oracle.e4m3_from_f32(x) == _nearest_even_encode(x), x
        assert oracle.e4m3_from_f32(-x) == _nearest_even_encode(-x), -x


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 448.0 / 448.0, 4.1 / 448.0, 1e-3, 7.7e-5, 1e-40])
def test_division_is_ieee_binary32(scale):
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(3000).astype(np.float32)
    s = np.float32(scale)
    with np.errstate(over="ignore", divide="ignore"):
        ref = xs / s
    got = np.array([oracle.div_f32(x, s) for x in xs], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _random_pool(rng, nb, hkv, bs, d, nan_frac=0.05):
    vals = (rng.standard_normal((nb, hkv, bs, d)) * rng.choice([1e-3, 0.3, 2.0, 50.0], size=(nb, hkv, 1, 1)))
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits = bits.copy()
    bits.reshape(-1)[rng.random(bits.size) < nan_frac] = 0x7FC0  # poisoned slots
    return bits


def test_quantize_pool_vs_torch_cast_and_kv_append():
    """orc_e4m3_quantize_pool (the quantised history both sides start from):
    every element equals torch's float8_e4m3fn cast of the fp32 quotient
    x / scale[block, head] (the scale of its own block and head, with scales of
    the amax / 448 form plus a few arbitrary ones), NaN slots give a NaN code,
    and the whole pool equals writing every token through the oracle's
    kv_append into an empty E4M3 cache."""
    rng = np.random.default_rng(21)
    nb, hkv, bs, d = 13, 3, 16, 64
    bits = _random_pool(rng, nb, hkv, bs, d)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    amax = torch.nan_to_num(x, nan=0.0).abs().amax(dim=(2, 3))
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    sc[0, 1] = 0.37  # scales not tied to the content: saturating and tiny codes
    sc[5, 2] = 3.1e-5
    scn = sc.numpy().astype(np.float32)
    got = oracle.quantize_pool(bits, scn)
    q = x / sc[:, :, None, None]
    fin = torch.isfinite(q) & (q.abs() <= 448.0)
    ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    fin = fin.numpy()
    assert np.array_equal(got[fin], ref[fin])
    nan = torch.isnan(x).numpy()
    assert np.all((got[nan] & 0x7F) == 0x7F)
    big = ~fin & ~nan  # quotients beyond 448 saturate
    assert big.any() and np.all((got[big] & 0x7F) == 0x7E)
    # the same bytes through kv_append, one token (all heads) per slot
    cache_k = np.zeros((nb, hkv, bs, d), np.uint8)
    cache_v = np.zeros_like(cache_k)
    tok = bits.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)  # [slot][head][d]
    slots = np.arange(nb * bs, dtype=np.int64)
    oracle.kv_append(cache_k, cache_v, scn, scn, oracle.KV_E4M3, tok, tok, slots)
    assert np.array_equal(cache_k, got) and np.array_equal(cache_v, got)
