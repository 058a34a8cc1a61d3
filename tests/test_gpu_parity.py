"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle at
sizes the oracle finishes in seconds: several tiles, ragged tails, every
supported head size, block size, GQA group and KV type, plus the bitwise
properties (kv_append, gather, placement and prefix-sharing invariance,
determinism) and the error path."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_lse, assert_parity, forward, gpu_caches, run_step
from tests.helpers import bits16, bytes8, host_caches, lse_bounds, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _spec(hist, incr, hq=8, hkv=2, d=64, bs=16, dtype="bf16", cfg=21, **kw):
    return W.Spec("case", cfg, hq, hkv, d, bs, list(hist), list(incr), kv_dtype=dtype, **kw)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("spec", [
    W.tiny(),
    _spec([40, 0, 17, 5], [9, 12, 1, 0]),
    _spec([100, 3], [70, 200], hq=32, hkv=8, d=128, bs=64),
])
def test_kv_append_bf16_bitwise(palib, spec):
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    kc_ref, vc_ref = host[0].copy(), host[1].copy()
    oracle.kv_append(kc_ref, vc_ref, None, None, oracle.KV_BF16, bits16(b.k_new), bits16(b.v_new),
                     b.slot_mapping.cpu().numpy())
    k, v, ks, vs = gpu_caches(b)
    palib.kv_append(palib.make_cache(k, v), b.k_new, b.v_new, b.slot_mapping)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(k), kc_ref) and np.array_equal(bits16(v), vc_ref)


def test_kv_append_skips_negative_slots(palib):
    b = W.make_batch(_spec([30], [20]), DEV)
    k, v, _, _ = gpu_caches(b)
    before = bits16(k).copy()
    slots = b.slot_mapping.clone()
    slots[::2] = -1
    palib.kv_append(palib.make_cache(k, v), b.k_new, b.v_new, slots)
    kc_ref, vc_ref = before.copy(), bits16(v).copy()
    torch.cuda.synchronize()
    oracle.kv_append(kc_ref, bits16(b.v_pool).copy(), None, None, 0, bits16(b.k_new),
                     bits16(b.v_new), slots.cpu().numpy())
    assert np.array_equal(bits16(k), kc_ref)


def test_kv_append_e4m3_every_bf16_pattern(palib):
    """All 65,536 bf16 bit patterns through the quantising append, under
    several per-block scales, bit-exact against the oracle's encoder."""
    hkv, d, bs = 1, 64, 16
    T = 65536 // (hkv * d)  # 1024 tokens -> 64 blocks
    pats = np.arange(65536, dtype=np.uint16)
    k_new = torch.from_numpy(pats.view(np.int16).reshape(T, hkv, d)).view(torch.bfloat16).to(DEV)
    v_new = torch.from_numpy(pats[::-1].copy().view(np.int16).reshape(T, hkv, d)).view(torch.bfloat16).to(DEV)
    nb = T // bs
    scale_set = np.float32([1.0, 0.5, 3.0, 1e-3, 4.1 / 448, 2.0 ** -7, 7.7e-5, 1.0 / 448, 300.0,
                            0.0125, 2.0 ** 20, 1.7e-2, 1.0, 0.25, 6.0, 0.9])
    rng = np.random.default_rng(5)
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    for trial in range(3):
        ks = rng.choice(scale_set, size=(nb, hkv)).astype(np.float32)
        vs = rng.choice(scale_set, size=(nb, hkv)).astype(np.float32)
        kc = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8, device=DEV)
        vc = torch.zeros_like(kc)
        palib.kv_append(palib.make_cache(kc, vc, torch.from_numpy(ks).to(DEV),
                                         torch.from_numpy(vs).to(DEV)), k_new, v_new, slots)
        kr = np.zeros((nb, hkv, bs, d), np.uint8)
        vr = np.zeros_like(kr)
        oracle.kv_append(kr, vr, ks, vs, oracle.KV_E4M3, bits16(k_new), bits16(v_new),
                         slots.cpu().numpy())
        torch.cuda.synchronize()
        gk, gv = bytes8(kc), bytes8(vc)
        # NaN inputs must give a NaN code (the sign of a NaN quotient is not
        # fixed by IEEE 754); every other input is compared bit for bit
        for got, ref, src in ((gk, kr, bits16(k_new)), (gv, vr, bits16(v_new))):
            src = src.reshape(got.shape)
            nan_in = ((src & 0x7F80) == 0x7F80) & ((src & 0x7F) != 0)
            assert np.all((got[nan_in] & 0x7F) == 0x7F)
            assert np.array_equal(got[~nan_in], ref[~nan_in]), int((got[~nan_in] != ref[~nan_in]).sum())


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_debug_gather_bitwise(palib, dtype):
    b = W.make_batch(_spec([77, 300], [3, 41], bs=16, dtype=dtype), DEV)
    host = host_caches(b)
    k, v, ks, vs = gpu_caches(b, host)
    c = palib.make_cache(k, v, ks, vs)
    for s in range(2):
        ctx = int(b.hist[s])
        bt_row = torch.from_numpy(b.block_tables[s]).to(DEV)
        ko = torch.empty((ctx, 2, 64), dtype=k.dtype, device=DEV)
        vo = torch.empty_like(ko)
        palib.pa_debug_gather(c, bt_row, ctx, ko, vo)
        torch.cuda.synchronize()
        ref_k = oracle.gather(host[0], b.block_tables[s], ctx)
        ref_v = oracle.gather(host[1], b.block_tables[s], ctx)
        view = (lambda t: bits16(t)) if dtype == "bf16" else bytes8
        assert np.array_equal(view(ko), ref_k) and np.array_equal(view(vo), ref_v)


# ---------------------------------------------------------------------------
def _needled(spec):
    """The spec with needles on the first and last new row of every sequence
    that has a history and new tokens."""
    nd = []
    for sq, (h, n) in enumerate(zip(spec.hist, spec.incr)):
        if h > 0 and n > 0:
            nd += sorted({(sq, 0), (sq, n - 1)})
    return W.with_needles(spec, needles=nd)


def check_against_oracle(palib, spec, want_lse=True, what=None, needles=True):
    spec = _needled(spec) if needles else spec
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    out, lse, c = run_step(palib, b, gpu_caches(b, host), want_lse=want_lse)
    torch.cuda.synchronize()
    ref, ref_lse, after = oracle_step(b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    fp8 = spec.kv_dtype == "e4m3"
    assert_parity(out, ref, fp8, what or spec.name, needles=[(r, h) for r, h, _, _ in b.needles])
    if want_lse:
        # per-path bars: exact-query kernels 2e-3; the 384-row prefill its
        # a-priori bound (tests/parity.py)
        assert_lse(lse, ref_lse, lse_bounds(b, after), what or spec.name)
    return b, out, c


def test_tiny_workload(palib):
    """1 session, 4 q / 1 KV head, d 64, 256 cached + 32 new tokens on a
    permuted 18-block table; then the decode of position 287 equals row 31."""
    b, out, c = check_against_oracle(palib, W.tiny(), what="tiny incremental")
    q_last = b.q[31:32].contiguous()
    out_dec, _ = forward(palib, b, c, q=q_last, hist=np.array([287], np.int32),
                         incr=np.array([1], np.int32))
    torch.cuda.synchronize()
    host = host_caches(b)
    oracle.kv_append(host[0], host[1], None, None, 0, bits16(b.k_new), bits16(b.v_new),
                     b.slot_mapping.cpu().numpy())
    ref, _ = oracle.attention(bits16(q_last), host[0], host[1], None, None, 0, b.block_tables,
                              [287], [1], 4, b.spec.scale)
    assert_parity(out_dec, ref, False, "tiny decode at 287")


CASES = [
    # (hist, incr, hq, hkv, d, bs, dtype)
    ([0], [300], 8, 2, 64, 16, "bf16"),                  # initial prefill, ragged tile
    ([1000], [130], 32, 8, 128, 16, "bf16"),              # incremental, 5 tiles
    ([1000, 513, 0, 64], [1, 1, 1, 1], 32, 8, 128, 16, "bf16"),  # decode batch
    ([2047, 40, 700], [2, 3, 4], 32, 8, 128, 64, "bf16"),  # short increments (decode kernel)
    ([333, 0, 4000, 7], [37, 129, 1, 260], 16, 16, 64, 16, "bf16"),  # group 1
    ([500, 90], [45, 3], 32, 16, 128, 16, "bf16"),        # group 2
    ([900, 31], [50, 6], 64, 8, 64, 64, "bf16"),          # group 8
    ([1200, 17, 64], [40, 1, 9], 16, 1, 128, 16, "bf16"),  # group 16
    ([1500, 20], [400, 7], 8, 8, 128, 64, "bf16"),        # group 1, d 128: 384-token tiles
    ([0, 2500], [700, 33], 64, 8, 128, 16, "bf16"),       # group 8, d 128: 48-token tiles
    ([640], [200], 32, 8, 128, 64, "e4m3"),              # E4M3, block 64
    ([900, 5000], [77, 1], 32, 8, 128, 16, "e4m3"),      # E4M3, block 16
    ([3000, 100], [1, 65], 8, 2, 64, 64, "e4m3"),        # E4M3, head dim 64
    ([20000, 3000, 50], [1, 1, 1], 32, 8, 128, 64, "e4m3"),  # E4M3 decode, split and merged
    ([9000, 130], [1, 3], 32, 8, 128, 16, "e4m3"),       # E4M3 decode, block 16
    ([7000, 33], [2, 1], 64, 8, 128, 16, "e4m3"),        # E4M3 decode, group 8
    ([4096, 0], [192, 97], 32, 8, 128, 16, "bf16"),       # whole 96-token tiles, step-aligned history
    ([8192], [384], 32, 8, 128, 64, "e4m3"),             # E4M3 prefill, whole tiles, block-aligned
    ([3000, 700], [250, 1], 32, 8, 128, 16, "bf16", 3.0),  # logit std 3 (q ~ N(0, 9))
    ([5000, 64], [130, 1], 32, 8, 128, 64, "e4m3", 3.0),   # logit std 3, E4M3
    ([2000, 90], [140, 2], 16, 4, 64, 16, "bf16", 3.0),    # logit std 3, head dim 64
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_small_configs(palib, case):
    hist, incr, hq, hkv, d, bs, dt = case[:7]
    q_std = case[7] if len(case) > 7 else 1.0
    print(f"[case] hist={hist} incr={incr} hq={hq} hkv={hkv} d={d} bs={bs} {dt} q_std={q_std}", flush=True)
    check_against_oracle(palib, _spec(hist, incr, hq, hkv, d, bs, dt, cfg=30 + CASES.index(case),
                                      q_std=q_std))


def _random_cases(n, seed=777):
    """Seeded random step shapes within the supported domain: 1-5 sequences
    mixing idle ones, decodes, short and multi-tile increments, histories up
    to a few thousand tokens, every head dim, block size, GQA group and KV type."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        k = int(rng.integers(1, 6))
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        hist = [int(rng.integers(0, 6000)) if rng.random() < 0.8 else 0 for _ in range(k)]
        incr = [int(rng.choice([0, 1, 1, 3, 17, 64, 200, 500])) for _ in range(k)]
        if sum(incr) == 0:
            incr[-1] = 1
        out.append((hist, incr, hkv * G, hkv, int(rng.choice([64, 128])), int(rng.choice([16, 64])),
                    str(rng.choice(["bf16", "e4m3"]))))
    return out


RANDOM_CASES = _random_cases(10)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"r{i}" for i in range(len(RANDOM_CASES))])
def test_random_configs(palib, case):
    hist, incr, hq, hkv, d, bs, dt = case
    print(f"[case] random hist={hist} incr={incr} hq={hq} hkv={hkv} d={d} bs={bs} {dt}", flush=True)
    check_against_oracle(palib, _spec(hist, incr, hq, hkv, d, bs, dt, cfg=200 + RANDOM_CASES.index(case)))


def test_long_decode_split_and_merge(palib):
    """A decode over 100K keys and an increment over 40K keys: both are cut
    into several items whose partials are merged."""
    spec = _spec([100_000, 40_000], [1, 300], 32, 8, 128, 16, "bf16", cfg=50)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    out, _, _ = run_step(palib, b, gpu_caches(b, host))
    torch.cuda.synchronize()
    rows = [0, 1, 2, 150, 299, 300]
    ref, _, _ = oracle_step(b, rows=rows, caches=host)
    assert_parity(out[rows], ref, False, "long decode + increment (sampled rows)")


# ---------------------------------------------------------------------------
def test_placement_invariance_bitwise(palib):
    s1 = _spec([700, 61, 0], [5, 1, 140], 32, 8, 128, 16, perm_seed=0, cfg=60)
    s2 = _spec([700, 61, 0], [5, 1, 140], 32, 8, 128, 16, perm_seed=9, cfg=60)
    outs = []
    for s in (s1, s2):
        b = W.make_batch(s, DEV)
        out, _, _ = run_step(palib, b, gpu_caches(b))
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_shared_prefix_equals_unshared_bitwise(palib):
    spec = _spec([3000, 2500, 4100], [1, 1, 1], 32, 8, 128, 16, shared_prefix_tokens=1024,
                 shared_seqs=[0, 1, 2], cfg=61)
    b = W.make_batch(spec, DEV)
    k, v, _, _ = gpu_caches(b)
    out_sh, _, c = run_step(palib, b, (k, v, None, None))
    # copies of the 64 shared blocks for sequences 1 and 2
    nb = k.shape[0]
    shared = torch.from_numpy(b.block_tables[0, :64].astype(np.int64)).to(DEV)
    k2 = torch.cat([k, k[shared], k[shared]])
    v2 = torch.cat([v, v[shared], v[shared]])
    bt2 = b.block_tables.copy()
    bt2[1, :64] = np.arange(nb, nb + 64)
    bt2[2, :64] = np.arange(nb + 64, nb + 128)
    b.block_tables = bt2
    out_un, _ = forward(palib, b, palib.make_cache(k2, v2))
    torch.cuda.synchronize()
    assert torch.equal(out_sh.view(torch.int16), out_un.view(torch.int16))


def test_deterministic(palib):
    b = W.make_batch(_spec([5000, 30], [200, 1], 32, 8, 128, 16, cfg=62), DEV)
    k, v, _, _ = gpu_caches(b)
    out1, _, c = run_step(palib, b, (k, v, None, None))
    out2, _ = forward(palib, b, c)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_idle_sequences_and_empty_step(palib):
    spec = _spec([50, 80, 0, 30], [0, 7, 0, 1], cfg=63)
    check_against_oracle(palib, spec, what="idle sequences")
    b = W.make_batch(_spec([50], [0], cfg=64), DEV)
    c = palib.make_cache(b.k_pool, b.v_pool)
    out = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    palib.paged_attn_forward(b.q, c, torch.from_numpy(b.block_tables).to(DEV), b.hist, b.incr,
                             b.spec.scale, out, ws)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping.to(DEV))
    torch.cuda.synchronize()


def test_error_path_writes_nothing(palib):
    b = W.make_batch(_spec([100], [10], cfg=65), DEV)
    c = palib.make_cache(b.k_pool, b.v_pool)
    out = torch.full((10, 8, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(palib.PagedAttnError) as e:
        palib.paged_attn_forward(b.q, c, torch.from_numpy(b.block_tables).to(DEV), b.hist, b.incr,
                                 b.spec.scale, out, ws)
    assert e.value.status == palib.PA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_measurement_hooks(palib):
    """The ceiling kernels bench.py times: the streaming read touches every
    32-bit word of the buffer exactly once (the XOR of its per-thread
    checksums is the XOR of the buffer), and the MFMA loop's accumulators
    equal iters times one product of its constant operands."""
    print("[case] measurement hooks", flush=True)
    n = (1 << 20) + 3 * 4096  # whole 4 KB segments, not a multiple of the grid's waves
    g = torch.Generator(device="cpu").manual_seed(5)
    words = torch.randint(0, 1 << 31, (n // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = words.to(DEV)
    outr = torch.empty(palib.PEAK_READ_THREADS, dtype=torch.int32, device=DEV)
    palib.pa_peak_read(buf, outr)
    torch.cuda.synchronize()
    x = np.bitwise_xor.reduce(outr.cpu().numpy().astype(np.uint32))
    assert x == np.bitwise_xor.reduce(words.numpy().astype(np.uint32))
    out = torch.empty(palib.PEAK_MFMA_THREADS, dtype=torch.float32, device=DEV)
    palib.pa_peak_mfma(out, 3)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o)) and o.min() > 0
    # every MFMA adds the same product: twice the iterations give twice the sums (exact)
    o2 = torch.empty_like(out)
    palib.pa_peak_mfma(o2, 6)
    torch.cuda.synchronize()
    assert np.allclose(o2.cpu().numpy(), 2 * o, rtol=1e-6)
    with pytest.raises(palib.PagedAttnError):
        palib.pa_peak_mfma(out, 0)


def test_xcd_dispatch_is_round_robin(palib):
    """The planner's L2 locality plan assumes that the work-groups w of a
    launch with equal w mod num_xcds run on one XCD, the num_xcds classes on
    distinct XCDs (work-group w on XCD (w + k) mod num_xcds; k is 0 for a
    launch alone on the GPU and can differ while another stream's launch is
    being dispatched): check where 4,096 work-groups actually ran."""
    cus, xcds = palib.pa_device_shape()
    print(f"[case] device shape: {cus} CUs, {xcds} XCDs", flush=True)
    out = torch.full((4096,), -1, dtype=torch.int32, device=DEV)
    palib.pa_debug_xcc_ids(out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    k = int(got[0]) % xcds
    want = (np.arange(got.size) + k) % xcds
    match = float(np.mean(got == want))
    print(f"[xcd] round-robin match {match:.4f} (offset {k}); first ids {got[:16].tolist()}", flush=True)
    assert np.all(got >= 0) and match >= 0.99
