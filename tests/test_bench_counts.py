"""The benchmark's algorithmic work counts (CPU only).

bench.py turns kernel times into TFLOP/s and GB/s with `prefill_flops` and
`decode_bytes`.  These tests check them against counts worked out by hand from
the definitions: 4 * d * Hq flops per unmasked (query, key) pair (QK^T and PV,
a multiply and an add each), and 2 * Hkv * d * elem bytes of K and V per
context token.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_prefill_flops_headline():
    # 2,700 new tokens over 45,700 cached: each new token i (0-based) sees
    # 45,700 + i + 1 keys
    pairs = sum(45_700 + i + 1 for i in range(2_700))
    assert pairs == 2_700 * 45_700 + 2_700 * 2_701 // 2
    fl = bench.prefill_flops([45_700], [2_700], 32, 128)
    assert fl == 4 * 128 * 32 * pairs
    assert abs(fl / 1e12 - 2.081) < 0.001


def test_prefill_flops_other_points():
    assert abs(bench.prefill_flops([0], [45_700], 32, 128) / 1e12 - 17.109) < 0.001
    assert abs(bench.prefill_flops([131_072], [2_700], 32, 128) / 1e12 - 5.858) < 0.001
    assert abs(bench.prefill_flops([1_044_480], [4_096], 32, 128) / 1e12 - 70.23) < 0.01
    # a decode row is one pair per context token
    assert bench.prefill_flops([99], [1], 4, 64) == 4 * 64 * 4 * 100


def test_decode_bytes_long_context_step():
    # context 1,048,576 in E4M3: 2 * 8 * 128 bytes per token, plus q and out
    # (32 heads * 128 * 2 bytes each) and one 4-byte block id per 64 tokens
    spec = W.Spec("x", 5, 32, 8, 128, 64, [1_048_575], [1], kv_dtype="e4m3")
    b = bench.decode_bytes(spec)
    assert b == 1_048_576 * 2048 + 2 * 32 * 128 * 2 + (1_048_576 // 64) * 4
    assert abs(b / 1e9 - 2.148) < 0.001


def test_decode_bytes_batch():
    spec = W.decode_batch()
    ctx = [h + 1 for h in spec.hist]
    nb = sum(-(-c // 16) for c in ctx)
    assert bench.decode_bytes(spec) == sum(ctx) * 4096 + 2 * 64 * 32 * 128 * 2 + nb * 4


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; a request for more exits with a message."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_mixed_step_split():
    """The mixed step's parts: prefill flops over the four increments only,
    decode bytes over the 48 decodes with the 10,000-token shared prefix
    counted once."""
    spec = W.mixed()
    fl, dfl, byts = bench.mixed_parts(spec)
    pre = [i for i, n in enumerate(spec.incr) if n > 1]
    dec = [i for i, n in enumerate(spec.incr) if n == 1]
    assert len(pre) == 4 and len(dec) == 48
    pairs = sum(spec.incr[i] * spec.hist[i] + spec.incr[i] * (spec.incr[i] + 1) // 2 for i in pre)
    assert fl == 4 * 128 * 32 * pairs
    assert dfl == 4 * 128 * 32 * sum(spec.hist[i] + 1 for i in dec)
    ctx = sum(spec.hist[i] + 1 for i in dec)
    assert byts == (ctx - 7 * 10_000) * 4096 + 2 * 48 * 32 * 128 * 2
