"""GPU parity of the 4-bit (OCP MXFP4) KV path against the oracle: the
device's widening of every (code byte, scale byte) pair, the quantising
kv_append bit for bit (every bf16 pattern, special groups, random slots over
caches whose unwritten bytes are garbage), and attention over MXFP4 caches
(decode and short increments, every GQA group, both block sizes, ragged
lengths whose last blocks hold unwritten slots with NaN scales, split items,
needles, large-variance queries, the 1M-token session).  The widened values
are exact in bf16, so the bars are the bf16 path's."""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, forward, gpu_caches
from tests.helpers import bits16, bytes8, host_caches
from tests.test_gpu_parity import check_against_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _spec(hist, incr, hq=32, hkv=8, bs=16, cfg=41, **kw):
    return W.Spec("mxfp4", cfg, hq, hkv, 128, bs, list(hist), list(incr), kv_dtype="mxfp4", **kw)


def _bf16_bits_equal(got_bf16: torch.Tensor, ref: np.ndarray):
    """bf16 device values equal to fp64 oracle values that bf16 holds exactly
    (NaN where the oracle has NaN, the sign of zero included).  Values past
    bf16's range (a code of 4 or 6 under scale bytes 253 and 254, which the
    encoder never writes) overflow to an infinity of their sign."""
    g = bits16(got_bf16).reshape(-1)
    r = ref.reshape(-1)
    nan = np.isnan(r)
    gnan = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    assert np.array_equal(gnan, nan)
    big = ~nan & (np.abs(np.nan_to_num(r)) > 3.3895313892515355e38)
    assert np.array_equal(g[big], np.where(r[big] > 0, 0x7F80, 0xFF80).astype(np.uint16))
    fin = ~nan & ~big
    rb = torch.from_numpy(r[fin]).to(torch.bfloat16)
    assert torch.equal(rb.to(torch.float64), torch.from_numpy(r[fin])), "oracle values not exact in bf16"
    assert np.array_equal(g[fin], rb.view(torch.int16).numpy().view(np.uint16))


def test_widening_every_code_and_scale_byte(palib):
    """Token t, group j of a 1,024-token sequence holds scale byte (4t + j) %
    256 and the 16 code bytes 16 ((4t + j) // 256) .. +15: every (code byte,
    scale byte) pair once, scale bytes 0 (2^-127), 254 and 255 (NaN)
    included; pa_debug_gather widens them with the attention kernels'
    conversion."""
    nb, hkv, bs, d, ctx = 64, 1, 16, 128, 1024
    rng = np.random.default_rng(12)
    perm = rng.permutation(nb).astype(np.int32)
    kc = np.zeros((nb, hkv, bs, d // 2), np.uint8)
    ks = np.zeros((nb, hkv, d // 32, bs), np.uint8)
    for t in range(ctx):
        blk, off = perm[t // bs], t % bs
        for j in range(4):
            combo = 4 * t + j
            ks[blk, 0, j, off] = combo % 256
            kc[blk, 0, off, 16 * j:16 * j + 16] = np.arange(16 * (combo // 256), 16 * (combo // 256) + 16)
    vc, vs = kc[::-1].copy(), ks[::-1].copy()  # V: the same pairs on other blocks
    dk = [torch.from_numpy(x).to(DEV) for x in (kc, vc, ks, vs)]
    c = palib.make_cache(*dk)
    bt = torch.from_numpy(perm).to(DEV)
    ko = torch.empty((ctx, hkv, d), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty_like(ko)
    palib.pa_debug_gather(c, bt, ctx, ko, vo)
    torch.cuda.synchronize()
    _bf16_bits_equal(ko, oracle.gather_values(kc, ks, oracle.KV_MXFP4, perm, ctx))
    _bf16_bits_equal(vo, oracle.gather_values(vc, vs, oracle.KV_MXFP4, perm, ctx))


def _garbage_caches(nb, hkv, bs, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, (nb, hkv, bs, d // 2), dtype=np.uint8),
            rng.integers(0, 256, (nb, hkv, bs, d // 2), dtype=np.uint8),
            rng.integers(0, 256, (nb, hkv, d // 32, bs), dtype=np.uint8),
            rng.integers(0, 256, (nb, hkv, d // 32, bs), dtype=np.uint8))


def _append_both(palib, caches, k_new, v_new, slots):
    host = [x.copy() for x in caches]
    dev = [torch.from_numpy(x).to(DEV) for x in caches]
    palib.kv_append(palib.make_cache(*dev), k_new, v_new, slots)
    oracle.kv_append(host[0], host[1], host[2], host[3], oracle.KV_MXFP4, bits16(k_new), bits16(v_new),
                     slots.cpu().numpy())
    torch.cuda.synchronize()
    for g, h, name in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        got = bytes8(g)
        assert np.array_equal(got, h), f"{name}: {int((got != h).sum())} bytes differ"


def test_append_every_bf16_pattern(palib):
    """All 65,536 bf16 patterns in 32-element groups (in order for K,
    permuted for V): groups with a NaN or an infinity, subnormal and
    zero groups, saturation."""
    hkv, d, bs = 1, 128, 16
    T = 65536 // d
    pats = np.arange(65536, dtype=np.uint16)
    rng = np.random.default_rng(1)
    for trial in range(2):
        kp = pats if trial == 0 else rng.permutation(pats)
        vp = rng.permutation(pats)
        k_new = torch.from_numpy(kp.view(np.int16).reshape(T, hkv, d).copy()).view(torch.bfloat16).to(DEV)
        v_new = torch.from_numpy(vp.view(np.int16).reshape(T, hkv, d).copy()).view(torch.bfloat16).to(DEV)
        slots = torch.from_numpy(rng.permutation(T).astype(np.int64)).to(DEV)
        _append_both(palib, _garbage_caches(T // bs, hkv, bs, d, trial), k_new, v_new, slots)


@pytest.mark.parametrize("bs", [16, 64])
def test_append_random_groups_and_skipped_slots(palib, bs):
    """Groups of every magnitude (std 10^-30 .. 10^30, exact zeros, one
    element dominant), 8 KV heads, random slots with some skipped; bytes of
    unnamed slots keep their garbage."""
    hkv, d, T = 8, 128, 700
    rng = np.random.default_rng(bs)
    mag = 10.0 ** rng.uniform(-30, 30, size=(T, hkv, d // 32, 1))
    x = rng.standard_normal((T, hkv, d // 32, 32)) * mag
    x[rng.random((T, hkv, d // 32)) < 0.05] = 0.0
    spike = rng.random((T, hkv, d // 32)) < 0.1
    x[spike, 0] *= 1e3
    k_new = torch.from_numpy(x.reshape(T, hkv, d)).to(torch.bfloat16).to(DEV)
    v_new = torch.from_numpy((x[::-1] * 0.5).reshape(T, hkv, d).copy()).to(torch.bfloat16).to(DEV)
    nb = 2 * T // bs + 3
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.1] = -1
    _append_both(palib, _garbage_caches(nb, hkv, bs, d, 7), k_new, v_new, torch.from_numpy(slots).to(DEV))


# ---------------------------------------------------------------------------
# attention: decode-class steps (tokens x G <= 16 per sequence)
CASES = {
    "g4_bs16": _spec([100, 1000, 37, 4000, 0], [1, 1, 1, 1, 1]),
    "g4_bs64": _spec([100, 1000, 37, 4000], [1, 1, 1, 1], bs=64),
    "g1": _spec([333, 64, 2049], [1, 1, 1], hq=8, hkv=8),
    "g2_inc8": _spec([500, 77], [8, 3], hq=16, hkv=8),
    "g8_inc2": _spec([1500, 10, 640], [2, 1, 2], hq=32, hkv=4, bs=64),
    "g16": _spec([901, 5], [1, 1], hq=32, hkv=2),
    "g1_inc16": _spec([1000], [16], hq=4, hkv=4),
    "long_split": _spec([70_000, 33_333], [1, 4]),
    "long_split_bs64": _spec([70_001], [1], bs=64),
    "q_std3": _spec([3000, 12_000], [1, 1], q_std=3.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(palib, name):
    print(f"[case] mxfp4 {name}", flush=True)
    check_against_oracle(palib, CASES[name], what=f"mxfp4 {name}")


@pytest.mark.parametrize("needled", [False, True], ids=["plain", "needles"])
def test_long_context_decode(palib, needled):
    """One decode at 1,048,576 keys over an MXFP4 cache (block 64), and a
    decode step after one more appended token."""
    spec = W.long_context_mxfp4(hist=1_048_575, incr=1, decode_steps=1)
    if needled:
        spec = W.with_needles(spec, needles=[(0, 0)], decode_steps=[1])
    print(f"[case] long_context_mxfp4 decode needled={needled}", flush=True)
    b = W.make_batch(spec, DEV)
    t = time.time()
    host = host_caches(b)
    print(f"[oracle] encoded the pool in {time.time() - t:.1f}s", flush=True)
    caches = gpu_caches(b, host)
    c = palib.make_cache(*caches)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    out, _ = forward(palib, b, c)
    kc, vc, ks, vs, dt = host
    oracle.kv_append(kc, vc, ks, vs, dt, bits16(b.k_new), bits16(b.v_new), b.slot_mapping.cpu().numpy())
    torch.cuda.synchronize()
    for g, h in zip(caches, (kc, vc, ks, vs)):
        assert torch.equal(g.cpu(), torch.from_numpy(h))
    ref, _ = oracle.attention(bits16(b.q), kc, vc, ks, vs, dt, b.block_tables, b.hist, b.incr, 32, spec.scale)
    nd = [(r, h) for r, h, _, _ in b.needles]
    assert_parity(out, ref, False, "long_context_mxfp4 decode", needles=nd)
    # one more step: append token 1,048,576 and attend
    q, k1, v1 = W.decode_step_tokens(spec, 1, DEV)
    pos = 1_048_576
    slot = torch.tensor([W.slot_of(b, 0, pos)], dtype=torch.int64, device=DEV)
    palib.kv_append(c, k1, v1, slot)
    outd, _ = forward(palib, b, c, q=q, hist=np.array([pos], np.int32), incr=np.array([1], np.int32))
    oracle.kv_append(kc, vc, ks, vs, dt, bits16(k1), bits16(v1), slot.cpu().numpy())
    torch.cuda.synchronize()
    refd, _ = oracle.attention(bits16(q), kc, vc, ks, vs, dt, b.block_tables, [pos], [1], 32, spec.scale)
    ndd = [(0, b.decode_needles[1][0])] if 1 in b.decode_needles else []
    assert_parity(outd, refd, False, "long_context_mxfp4 decode step 1", needles=ndd)


# ---------------------------------------------------------------------------
# attention: prefill tiles (the 384-row kernel with MXFP4 widening), mixed steps
PREFILL_CASES = {
    "initial_bs16": _spec([0], [1000]),
    "incremental_bs16": _spec([2000, 37], [700, 400]),
    "incremental_bs64": _spec([4100], [900], bs=64),
    "ragged_g8": _spec([333, 0], [150, 97], hq=32, hkv=4),
    "g1": _spec([1200], [300], hq=8, hkv=8),
    "g16_bs64": _spec([640], [130], hq=32, hkv=2, bs=64),
    "mixed": _spec([5000, 900, 12_000, 0, 77], [600, 1, 1, 300, 1]),
    "long_split": _spec([60_000], [400], bs=64),
    "q_std3": _spec([3000], [500], q_std=3.0),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_parity(palib, name):
    print(f"[case] mxfp4 prefill {name}", flush=True)
    check_against_oracle(palib, PREFILL_CASES[name], what=f"mxfp4 prefill {name}")


@pytest.mark.parametrize("needled", [False, True], ids=["plain", "needles"])
def test_long_context_prefill(palib, needled):
    """The 4,096-token incremental prefill over the 1,044,480-token MXFP4
    history (block 64): sampled rows at the planner's tile boundaries, the
    cache after the quantising append byte for byte."""
    from tests.test_gpu_fullsize import local_needles, plan_tiles, tile_boundary_rows
    spec = W.long_context_mxfp4()
    tiles = plan_tiles(palib, spec)
    rows = tile_boundary_rows(tiles, 0, spec.incr[0], np.random.default_rng(4), k=2)
    if needled:
        spec = W.with_needles(spec, needles=[(0, r) for r in rows[::2]])
    print(f"[case] long_context_mxfp4 prefill needled={needled} rows={rows}", flush=True)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    caches = gpu_caches(b, host)
    c = palib.make_cache(*caches)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    out, _ = forward(palib, b, c)
    kc, vc, ks, vs, dt = host
    oracle.kv_append(kc, vc, ks, vs, dt, bits16(b.k_new), bits16(b.v_new), b.slot_mapping.cpu().numpy())
    torch.cuda.synchronize()
    for g, h in zip(caches, (kc, vc, ks, vs)):
        assert torch.equal(g.cpu(), torch.from_numpy(h))
    t = time.time()
    ref, _ = oracle.attention(bits16(b.q), kc, vc, ks, vs, dt, b.block_tables, b.hist, b.incr, 32, spec.scale,
                              rows=rows)
    print(f"[oracle] prefill rows in {time.time() - t:.1f}s", flush=True)
    assert_parity(out[rows], ref, False, "long_context_mxfp4 prefill", needles=local_needles(b, rows))
