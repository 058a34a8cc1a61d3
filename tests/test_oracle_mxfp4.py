"""Pins for the oracle's MXFP4 codec, kv_append and element access (CPU only).

E2M1 decoding is checked against the format's published table
(tests/golden/mxfp4_format.txt, from the OCP MX specification), E8M0 against
torch's float8_e8m0fnu conversion; the encoder (nearest value, ties to the
even mantissa, saturation; shared exponent floor(log2 amax) - emax) against
an exact brute-force search written here with Python fractions; kv_append
against an independent packing of those codes; the attention and value
gather on an MXFP4 cache against the same computation on a bf16 cache that
holds the decoded values (which bf16 represents exactly).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.txt")


def _golden():
    e2m1, e8m0, emax = {}, {}, None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "e2m1":
            e2m1[int(f[1], 16)] = float(f[2])
        elif f[0] == "e8m0":
            e8m0[int(f[1])] = float("nan") if f[2] == "nan" else 2.0 ** int(f[2].split("^")[1])
        elif f[0] == "emax_e2m1":
            emax = int(f[1])
    return e2m1, e8m0, emax


E2M1, E8M0, EMAX = _golden()
MAGS = [Fraction(E2M1[c]) for c in range(8)]


def test_e2m1_decode_matches_published_table():
    assert len(E2M1) == 16
    for c in range(16):
        got = oracle.e2m1_to_f64(c)
        assert got == E2M1[c] and math.copysign(1, got) == math.copysign(1, E2M1[c]), c
    # only the low 4 bits are a code
    assert all(oracle.e2m1_to_f64(c | 0xF0) == oracle.e2m1_to_f64(c) for c in range(16))


def test_e8m0_decode_vs_torch_and_table():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_to_f64(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    for b, v in E8M0.items():
        assert (np.isnan(v) and np.isnan(got[b])) or got[b] == v


def _brute_e2m1(v: Fraction, neg: bool) -> int:
    """Nearest magnitude; ties to the even mantissa (code bit 0 clear);
    beyond 6 saturate."""
    a = abs(v)
    if a >= MAGS[7]:
        code = 7
    else:
        d = [abs(m - a) for m in MAGS]
        best = [c for c in range(8) if d[c] == min(d)]
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
    return code | (8 if neg else 0)


def _bf16_values(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_e2m1_encode_vs_brute_force_all_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint16)
    vals = _bf16_values(bits)
    sel = np.isfinite(vals) & (np.abs(vals) <= 16.0)
    for x in vals[sel]:
        want = _brute_e2m1(Fraction(float(x)), bool(np.signbit(x)))
        assert oracle.e2m1_from_f64(float(x)) == want, x


def test_e2m1_encode_ties_and_saturation():
    cases = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6,
             5.0001: 0x7, 6.0: 0x7, 7.99: 0x7, 1e30: 0x7, -0.25: 0x8, -5.0: 0xE, -0.0: 0x8}
    for v, c in cases.items():
        assert oracle.e2m1_from_f64(v) == c, v


def _brute_scale_byte(amax: float) -> int:
    if amax == 0.0:
        return 0
    k = -200
    while Fraction(2) ** (k + 1) <= Fraction(amax):
        k += 1
    assert Fraction(2) ** k <= Fraction(amax) < Fraction(2) ** (k + 1)
    return min(max(k - EMAX + 127, 0), 254)


def test_scale_byte_vs_brute_force():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)  # positive finite bf16, strided
    for a in list(_bf16_values(bits)) + [0.0, 2.0 ** -133, 2.0 ** -125, 3.0 * 2 ** 126]:
        assert oracle.mxfp4_scale_byte(float(a)) == _brute_scale_byte(float(a)), a


def _brute_group(vals):
    if not np.all(np.isfinite(vals)):
        return [0] * len(vals), 0xFF
    sb = _brute_scale_byte(float(np.max(np.abs(vals))))
    X = Fraction(2) ** (sb - 127)
    return [_brute_e2m1(Fraction(float(v)) / X, bool(np.signbit(v))) for v in vals], sb


def _bits_of(vals):
    return torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed", range(6))
def test_group_encode_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    for trial in range(40):
        std = float(10.0 ** rng.uniform(-30, 30))
        v = rng.standard_normal(32) * std
        if trial % 5 == 0:
            v[rng.integers(32)] = 0.0
        if trial % 7 == 0:
            v[:] = 0.0
        bits = _bits_of(v)
        vals = _bf16_values(bits)
        codes, sb = oracle.mxfp4_encode_group(bits)
        want_codes, want_sb = _brute_group(vals)
        assert sb == want_sb and list(codes) == want_codes, (seed, trial)
        if sb not in (0, 0xFF):
            # the largest magnitude lands on 4 or 6 (rounding or saturating)
            top = max(abs(E2M1[c]) for c in codes)
            assert top in (4.0, 6.0)


def test_group_encode_non_finite():
    for bad in (float("nan"), float("inf"), float("-inf")):
        v = np.linspace(-3, 3, 32)
        v[5] = bad
        codes, sb = oracle.mxfp4_encode_group(_bits_of(v))
        assert sb == 0xFF and not codes.any()


def _mx_cache(nb, hkv, bs, d):
    return (np.zeros((nb, hkv, bs, d // 2), np.uint8), np.zeros((nb, hkv, bs, d // 2), np.uint8),
            np.zeros((nb, hkv, d // 32, bs), np.uint8), np.zeros((nb, hkv, d // 32, bs), np.uint8))


@pytest.mark.parametrize("bs,d", [(16, 128), (64, 64)])
def test_kv_append_mxfp4_vs_independent_packing(bs, d):
    rng = np.random.default_rng(bs + d)
    nb, hkv, T = 5, 2, 23
    kc, vc, ks, vs = _mx_cache(nb, hkv, bs, d)
    kc[:] = 0xAB
    ks[:] = 0x11
    k_new = _bits_of(rng.standard_normal((T, hkv, d)) * 3)
    v_new = _bits_of(rng.standard_normal((T, hkv, d)) * 0.01)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    oracle.kv_append(kc, vc, ks, vs, oracle.KV_MXFP4, k_new, v_new, slots)
    kv = _bf16_values(k_new)
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        blk, off = divmod(s, bs)
        for h in range(hkv):
            for grp in range(d // 32):
                codes, sb = _brute_group(kv[t, h, 32 * grp:32 * grp + 32])
                packed = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16)]
                assert list(kc[blk, h, off, 16 * grp:16 * grp + 16]) == packed
                assert ks[blk, h, grp, off] == sb
    written = np.zeros((nb, bs), bool)
    for s in slots[slots >= 0]:
        written[s // bs, s % bs] = True
    untouched = ~written
    assert np.all(kc.transpose(0, 2, 1, 3)[untouched] == 0xAB)
    assert np.all(ks.transpose(0, 3, 1, 2)[untouched] == 0x11)


def test_quantize_pool_equals_append():
    rng = np.random.default_rng(3)
    nb, hkv, bs, d = 4, 2, 16, 128
    src = _bits_of(rng.standard_normal((nb, hkv, bs, d)) * 2)
    codes, scales = oracle.mxfp4_quantize_pool(src)
    kc, vc, ks, vs = _mx_cache(nb, hkv, bs, d)
    toks = src.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    oracle.kv_append(kc, vc, ks, vs, oracle.KV_MXFP4, toks, toks, np.arange(nb * bs, dtype=np.int64))
    assert np.array_equal(codes, kc) and np.array_equal(scales, ks)


def _decoded_bf16_pool(codes, scales):
    nb, hkv, bs, half = codes.shape
    d = 2 * half
    lo, hi = codes & 0xF, codes >> 4
    el = np.empty((nb, hkv, bs, d), np.uint8)
    el[..., 0::2], el[..., 1::2] = lo, hi
    val = np.vectorize(lambda c: E2M1[int(c)])(el)
    sc = np.vectorize(lambda b: E8M0[int(b)] if int(b) in E8M0 else 2.0 ** (int(b) - 127))(scales)
    val = val * np.repeat(sc.transpose(0, 1, 3, 2), 32, axis=3)
    return _bits_of(val), val


def test_attention_on_mxfp4_equals_attention_on_decoded_bf16():
    rng = np.random.default_rng(8)
    nb, hkv, bs, d, hq = 12, 2, 16, 64, 8
    kc, ks = oracle.mxfp4_quantize_pool(_bits_of(rng.standard_normal((nb, hkv, bs, d))))
    vc, vs = oracle.mxfp4_quantize_pool(_bits_of(rng.standard_normal((nb, hkv, bs, d)) * 4))
    kb, kval = _decoded_bf16_pool(kc, ks)
    vb, _ = _decoded_bf16_pool(vc, vs)
    assert np.array_equal(_bf16_values(kb), kval)  # bf16 holds the decoded values exactly
    hist, incr = np.array([40, 0, 70], np.int32), np.array([9, 5, 1], np.int32)
    bt = np.stack([rng.permutation(nb)[:6] for _ in range(3)]).astype(np.int32)
    q = _bits_of(rng.standard_normal((int(incr.sum()), hq, d)))
    o4, l4 = oracle.attention(q, kc, vc, ks, vs, oracle.KV_MXFP4, bt, hist, incr, hq, 0.125)
    ob, lb = oracle.attention(q, kb, vb, None, None, oracle.KV_BF16, bt, hist, incr, hq, 0.125)
    assert np.array_equal(o4, ob) and np.array_equal(l4, lb)
    o4p, l4p = oracle.attention_partial(q[3, 1], kc, vc, ks, vs, oracle.KV_MXFP4, bt[0], 0, 43, 16, 40, 0.125)
    obp, lbp = oracle.attention_partial(q[3, 1], kb, vb, None, None, oracle.KV_BF16, bt[0], 0, 43, 16, 40, 0.125)
    assert np.array_equal(o4p, obp) and l4p == lbp
    g = oracle.gather_values(kc, ks, oracle.KV_MXFP4, bt[2], 71)
    want = kval[bt[2][np.arange(71) // bs], :, np.arange(71) % bs, :]
    assert np.array_equal(g, want)
