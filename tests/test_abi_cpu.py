"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, rejects every invalid argument on the host before touching
the device, and its work planner covers every (row, head, key) pair of the
causal pattern exactly once."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"PA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_exports_match_header(palib):
    names = declared_functions()
    assert set(names) == set(palib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", palib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(names), exported ^ set(names)
    for n in names:
        assert hasattr(palib.lib, n)


def test_product_path_does_not_reference_the_oracle(palib):
    pkg = os.path.join(ROOT, "paged_kv_cache_gqa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f
    out = subprocess.run(["ldd", palib.LIB_PATH], capture_output=True, text=True).stdout
    assert "liboracle" not in out


# ---------------------------------------------------------------------------
FAKE = 0x1000  # never dereferenced: every case below fails validation first


def cache(pa, **kw):
    c = dict(k_cache=FAKE, v_cache=FAKE, k_scale=None, v_scale=None, num_blocks=64,
             num_kv_heads=8, block_size=16, head_dim=128, dtype=pa.PA_KV_BF16)
    c.update(kw)
    return pa.pa_kv_cache(c["k_cache"], c["v_cache"], c["k_scale"], c["v_scale"], c["num_blocks"],
                          c["num_kv_heads"], c["block_size"], c["head_dim"], c["dtype"])


def fwd(pa, c, hist=(10,), incr=(5,), hq=32, max_blocks=4, scale=0.088, ws=FAKE,
        ws_bytes=1 << 30, q=FAKE, out=FAKE, bt=FAKE):
    h = np.asarray(hist, np.int32)
    n = np.asarray(incr, np.int32)
    return pa.lib.paged_attn_forward(q, C.byref(c), bt, max_blocks, h.ctypes.data_as(C.c_void_p),
                                     n.ctypes.data_as(C.c_void_p), len(h), hq, scale, out, None,
                                     ws, ws_bytes, None)


def test_forward_rejects_bad_arguments(palib):
    pa = palib
    E = pa
    cases = [
        (lambda: pa.lib.paged_attn_forward(FAKE, None, FAKE, 4, None, None, 0, 32, 0.1, FAKE, None,
                                           FAKE, 1, None), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa, head_dim=96)), E.PA_ERR_UNSUPPORTED),
        (lambda: fwd(pa, cache(pa, block_size=32)), E.PA_ERR_UNSUPPORTED),
        (lambda: fwd(pa, cache(pa, dtype=7)), E.PA_ERR_UNSUPPORTED),
        (lambda: fwd(pa, cache(pa, dtype=pa.PA_KV_FP8_E4M3)), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa, k_scale=FAKE, v_scale=FAKE)), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa, k_cache=None)), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa, num_blocks=0)), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), hq=30), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), hq=24), E.PA_ERR_UNSUPPORTED),   # group 3
        (lambda: fwd(pa, cache(pa, num_kv_heads=1), hq=32), E.PA_ERR_UNSUPPORTED),  # group 32
        (lambda: fwd(pa, cache(pa), hist=(-1,)), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), incr=(-3,)), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), hist=(60,), incr=(5,), max_blocks=4), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), scale=float("nan")), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), scale=float("inf")), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), scale=0.0), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), scale=-0.1), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), q=None), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa), out=None), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa), bt=None), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa), ws=None), E.PA_ERR_NULL_ARG),
        (lambda: fwd(pa, cache(pa), ws=FAKE + 8), E.PA_ERR_BAD_SHAPE),
        (lambda: fwd(pa, cache(pa), ws_bytes=16), E.PA_ERR_WORKSPACE_TOO_SMALL),
    ]
    for i, (call, want) in enumerate(cases):
        got = call()
        assert got == want, (i, got, want, pa.pa_last_error())
        assert pa.pa_last_error() != ""


def test_forward_with_no_rows_is_a_noop(palib):
    pa = palib
    assert fwd(pa, cache(pa), hist=(100, 7), incr=(0, 0), q=None, out=None, ws=None) == pa.PA_OK
    assert fwd(pa, cache(pa), hist=(), incr=(), q=None, out=None, ws=None) == pa.PA_OK


def test_kv_append_rejects_bad_arguments(palib):
    pa = palib
    c = cache(pa)
    assert pa.lib.kv_append(C.byref(c), None, FAKE, FAKE, 3, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.kv_append(C.byref(c), FAKE, FAKE, FAKE, -1, None) == pa.PA_ERR_BAD_SHAPE
    assert pa.lib.kv_append(None, FAKE, FAKE, FAKE, 3, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.kv_append(C.byref(cache(pa, head_dim=80)), FAKE, FAKE, FAKE, 3,
                            None) == pa.PA_ERR_UNSUPPORTED
    assert pa.lib.kv_append(C.byref(c), None, None, None, 0, None) == pa.PA_OK
    assert pa.lib.pa_debug_gather(C.byref(c), None, 5, FAKE, FAKE, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.pa_debug_gather(C.byref(c), FAKE, -5, FAKE, FAKE, None) == pa.PA_ERR_BAD_SHAPE
    assert pa.lib.pa_timing_read(9, None, None) == pa.PA_ERR_BAD_SHAPE


def test_workspace_size(palib):
    pa = palib
    c = cache(pa)
    small = pa.pa_workspace_size([100], [5], 32, c)
    assert small >= 256 and small % 256 == 0
    with pytest.raises(pa.PagedAttnError):
        pa.pa_workspace_size([100], [-5], 32, c)
    # a long decode is split: partial slots make the workspace larger
    big = pa.pa_workspace_size([1_000_000], [1], 32, c)
    assert big > 100 * small


# ---------------------------------------------------------------------------
def check_cover(pa, hist, incr, hq, hkv, d=128, bs=16):
    c = cache(pa, num_kv_heads=hkv, head_dim=d, block_size=bs)
    items, counts = pa.pa_debug_plan(hist, incr, hq, c)
    G = hq // hkv
    rowstart = np.concatenate([[0], np.cumsum(incr)])
    total_q = int(rowstart[-1])
    # coverage[row, kvh] = number of keys covered (must equal pos + 1, no overlaps)
    cover = {}
    parts = {}
    for idx, it in enumerate(items):
        seq, kvh, row0, pos0, nq, lo, hi, part = (int(x) for x in it)
        assert 0 <= kvh < hkv and nq >= 1 and nq * G <= (384 if d == 128 else 128)
        assert lo % 64 == 0 and hi > lo
        assert rowstart[seq] <= row0 and row0 + nq <= rowstart[seq] + incr[seq]
        assert pos0 == hist[seq] + (row0 - rowstart[seq])
        assert hi <= pos0 + nq  # never beyond the last row's key
        for r in range(row0, row0 + nq):
            cover.setdefault((r, kvh), []).append((lo, hi))
        if part >= 0:  # prefill and decode partials are separate slot arrays
            key = (idx < counts[0], part)
            parts[key] = parts.get(key, 0) + 1
    for r in range(total_q):
        seq = int(np.searchsorted(rowstart, r, side="right") - 1)
        pos = hist[seq] + (r - rowstart[seq])
        for kvh in range(hkv):
            rng = sorted(cover[(r, kvh)])
            assert rng[0][0] == 0
            for (a0, a1), (b0, b1) in zip(rng, rng[1:]):
                assert a1 == b0, (r, kvh, rng)  # contiguous, no overlap
            assert rng[-1][1] >= pos + 1
    assert all(v == 1 for v in parts.values())
    assert len(parts) == counts[3]
    if d == 128:
        # the persistent prefill never cuts a (tile, head) for length: a
        # partial slot per work-group boundary it crosses, at most
        units = {(int(it[2]), int(it[1])) for it in items[:counts[0]]}
        pre_parts = sum(1 for k in parts if k[0])
        assert pre_parts <= len(units) + 256, (pre_parts, len(units))
    return items, counts


def test_prefill_workspace_does_not_grow_with_context(palib):
    """An E4M3 incremental prefill of 4,096 tokens over 128K, 512K and 1M
    cached tokens: the work list and partials hold the same few slots (no
    per-context copy, no per-length cuts); coverage checked at 1M."""
    pa = palib
    c = cache(pa, dtype=pa.PA_KV_FP8_E4M3, k_scale=FAKE, v_scale=FAKE, block_size=64)
    sizes = [pa.pa_workspace_size([h], [4096], 32, c) for h in (131_072, 524_288, 1_044_480)]
    bound = (43 * 8 + 256) * 384 * (128 + 1) * 4 + (1 << 20)  # (units + boundaries) partials + list
    assert all(x <= bound for x in sizes), (sizes, bound)
    assert max(sizes) <= 1.05 * min(sizes), sizes
    check_cover(pa, [1_044_480], [4096], 32, 8, bs=64)


def test_planner_balances_persistent_prefill(palib):
    check_balance(palib, [0, 45_700, 3], [45_7, 2_700, 1], 32, 8)
    check_balance(palib, [131_072], [2_700], 32, 8)
    check_balance(palib, [100, 7, 999], [300, 200, 170], 16, 1)
    check_balance(palib, [1000, 70], [129, 300], 8, 8)
    check_balance(palib, [256], [32], 4, 1, d=64)                # register-staged kernel: none
    first = check_balance(palib, [0], [64], 4, 1)                # tiny: few work-groups
    assert 1 <= len(first) - 1 < 256


def test_planner_coschedules_mixed_steps(palib):
    """A head-dim-128 step with prefill and decode rows: the planner
    leaves a multiple of the XCD count of CUs (up to half) to the decode
    beside the prefill, cuts the prefill's ranges for the rest (balanced), and
    still covers the causal pattern exactly; steps with one kind of row, other
    KV types and the forced settings behave as documented."""
    import workloads as W
    cus, xcds = palib.pa_device_shape()
    m = W.mixed()
    c = cache(palib, num_kv_heads=8, head_dim=128, block_size=16)
    first = check_balance(palib, m.hist, m.incr, 32, 8)
    n_dec = cus - (len(first) - 1)
    assert 0 < n_dec <= cus // 2 and n_dec % xcds == 0, n_dec
    check_cover(palib, m.hist, m.incr, 32, 8)
    size_auto = palib.pa_workspace_size(m.hist, m.incr, 32, c)
    try:
        for force, want in ((0, cus), (20, cus - 16), (64, cus - 64), (1000, cus - cus // 2)):
            palib.pa_debug_overlap_cus(force)
            assert len(palib.pa_debug_plan_groups(m.hist, m.incr, 32, c)) - 1 == want, force
            check_balance(palib, m.hist, m.incr, 32, 8)
            check_cover(palib, m.hist, m.incr, 32, 8)
            assert palib.pa_workspace_size(m.hist, m.incr, 32, c) > 0
    finally:
        palib.pa_debug_overlap_cus(-1)
    assert palib.pa_workspace_size(m.hist, m.incr, 32, c) == size_auto
    # prefill only, decode only: nothing to co-schedule
    assert len(palib.pa_debug_plan_groups([45_700], [2_700], 32, c)) - 1 == cus
    # E4M3 and MXFP4 KV: fewer decode bytes and a slower decode per CU beside
    # the prefill, so no more CUs than bf16 (none for this step's short
    # decode); a prefill too small to hold every CU leaves the rest to the
    # decode in every format; the forced settings hold for both
    e4 = cache(palib, num_kv_heads=8, head_dim=128, block_size=64, dtype=palib.PA_KV_FP8_E4M3,
               k_scale=FAKE, v_scale=FAKE)
    f4 = cache(palib, num_kv_heads=8, head_dim=128, block_size=64, dtype=palib.PA_KV_MXFP4,
               k_scale=FAKE, v_scale=FAKE)
    small = ([3000, 900, 5000, 7000, 200, 40_000], [300, 150, 1, 1, 1, 1])
    n_small = cus - (len(palib.pa_debug_plan_groups(*small, 32, c)) - 1)
    assert n_small > cus // 2
    for q in (e4, f4):
        n_q = cus - (len(palib.pa_debug_plan_groups(m.hist, m.incr, 32, q)) - 1)
        assert 0 <= n_q <= n_dec and n_q % xcds == 0, n_q
        assert cus - (len(palib.pa_debug_plan_groups(*small, 32, q)) - 1) == n_small
        try:
            palib.pa_debug_overlap_cus(24)
            assert len(palib.pa_debug_plan_groups(m.hist, m.incr, 32, q)) - 1 == cus - 24
        finally:
            palib.pa_debug_overlap_cus(-1)
    # head_dim 64 (the register-staged kernels): no persistent prefill, no co-scheduling
    assert len(palib.pa_debug_plan_groups(m.hist, m.incr, 32, cache(palib, head_dim=64))) == 0


def test_planner_covers_causal_pattern_exactly(palib):
    check_cover(palib, [256], [32], 4, 1, d=64)                  # tiny workload
    check_cover(palib, [0, 45_700, 3], [45_7, 2_700, 1], 32, 8)  # mixed classes
    check_cover(palib, [131_072, 5, 0], [1, 1, 1], 32, 8)        # decode with splits
    check_cover(palib, [100, 7, 999], [3, 200, 17], 16, 1)       # group 16
    check_cover(palib, [1000, 70], [129, 300], 8, 8)             # group 1


def check_balance(pa, hist, incr, hq, hkv, d=128, bs=16):
    """Persistent prefill plan: each work-group's items are pieces of the
    flattened (KV head, tile, 64-key step) work, and every work-group gets
    the same number of steps to within one."""
    c = cache(pa, num_kv_heads=hkv, head_dim=d, block_size=bs)
    items, counts = pa.pa_debug_plan(hist, incr, hq, c)
    first = pa.pa_debug_plan_groups(hist, incr, hq, c)
    if d != 128:
        assert len(first) == 0
        return first
    G = hq // hkv
    pre = items[:counts[0]]
    assert len(first) >= 2 and first[0] == 0 and first[-1] == counts[0]
    assert np.all(np.diff(first) >= 1) and len(first) - 1 <= 256
    steps = []
    for w in range(len(first) - 1):
        tot = 0
        for it in pre[first[w]:first[w + 1]]:
            lo, hi = int(it[5]), int(it[6])
            assert int(it[4]) * G > 16
            tot += (hi + 63) // 64 - lo // 64
        steps.append(tot)
    assert max(steps) - min(steps) <= 1, (min(steps), max(steps))
    return first


def test_planner_splits_long_work_and_merges(palib):
    items, counts = check_cover(palib, [45_700], [2_700], 32, 8)
    assert counts[0] >= 29 * 8 and counts[2] > 0    # 29 tiles (96 tokens) x 8 heads, split
    first = check_balance(palib, [45_700], [2_700], 32, 8)
    assert len(first) - 1 == 256
    # (tile, head) units are split into a few key chunks plus the pieces cut
    # at work-group boundaries
    assert counts[3] <= 4 * 29 * 8 + 256
    items, counts = check_cover(palib, [1_048_575], [1], 32, 8, bs=64)
    assert counts[1] >= 256 and counts[2] == 8      # one long decode, split per head


def test_planner_initial_prefill_whole_tiles(palib):
    """Many tiles per KV head (an initial prefill): whole tiles go to the
    work-groups of the head's XCD (work-group w on XCD w % 8), longest first,
    with loads within 1% and no split tile."""
    hist, incr = [0], [45_700]
    items, counts = check_cover(palib, hist, incr, 32, 8)
    assert counts[2] == 0 and counts[3] == 0          # no merges, no partial slots
    c = cache(palib, num_kv_heads=8)
    first = palib.pa_debug_plan_groups(hist, incr, 32, c)
    assert len(first) - 1 == 256
    pre = items[:counts[0]]
    loads = []
    for w in range(256):
        its = pre[first[w]:first[w + 1]]
        assert np.all(its[:, 1] == w % 8)             # the XCD's KV head
        lens = its[:, 6] - its[:, 5]
        assert np.all(np.diff(lens) <= 0)             # longest first
        loads.append(int(lens.sum()))
    assert (max(loads) - min(loads)) / max(loads) < 0.01, (min(loads), max(loads))


def test_planner_random_configs(palib):
    """Seeded random step shapes (sequence count, history and increment
    lengths including idle sequences, decodes and multi-tile increments; every
    head dim, block size and GQA group): the work list covers every row's
    causal key range exactly once, partial slots are unique and merged, and
    the persistent prefill split stays balanced."""
    rng = np.random.default_rng(20261202)
    for trial in range(64):
        n = int(rng.integers(1, 9))
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        bs = int(rng.choice([16, 64]))
        hist = [int(rng.choice([0, 1, 63, 64, 1000, 20_000, 140_000])) + int(rng.integers(0, 97))
                for _ in range(n)]
        incr = [int(rng.choice([0, 1, 2, 5, 17, 96, 383, 1200])) for _ in range(n)]
        if sum(incr) == 0:
            incr[0] = 1
        print(f"[case] trial {trial}: hist={hist} incr={incr} hq={hkv * G} hkv={hkv} d={d} bs={bs}",
              flush=True)
        check_cover(palib, hist, incr, hkv * G, hkv, d=d, bs=bs)
        items, counts = palib.pa_debug_plan(hist, incr, hkv * G,
                                             cache(palib, num_kv_heads=hkv, head_dim=d, block_size=bs))
        if d == 128 and counts[0] > 0:
            check_balance(palib, hist, incr, hkv * G, hkv, d=d, bs=bs)


def test_measurement_hooks_reject_bad_arguments(palib):
    """Argument checks of the ceiling kernels run on the host, before any launch."""
    pa = palib
    assert pa.lib.pa_peak_mfma(None, 10, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.pa_peak_mfma(FAKE, 0, None) == pa.PA_ERR_BAD_SHAPE
    assert pa.lib.pa_peak_read(None, 4096, FAKE, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.pa_peak_read(FAKE, 4096, None, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.pa_peak_read(FAKE, 4096 + 16, FAKE, None) == pa.PA_ERR_BAD_SHAPE
    assert pa.lib.pa_peak_read(FAKE, 0, FAKE, None) == pa.PA_ERR_BAD_SHAPE
    assert "4096" in pa.pa_last_error()


# ---------------------------------------------------------------------------
# The binding's own checks: a tensor of the wrong dtype, shape, layout or
# device is refused before the library sees its pointer.  (Dtype, shape and
# layout are checked before the device, so CPU tensors reach every check.)
def _expect_bad(pa, fn, what):
    with pytest.raises(pa.PagedAttnError) as e:
        fn()
    assert what in str(e.value), str(e.value)


def test_binding_rejects_bad_tensors(palib):
    import torch
    pa = palib
    bf, i32, i64 = torch.bfloat16, torch.int32, torch.int64
    kc = torch.zeros((4, 2, 16, 64), dtype=bf)
    # caches
    _expect_bad(pa, lambda: pa.make_cache(kc.float(), kc.float()), "dtype")
    _expect_bad(pa, lambda: pa.make_cache(kc, kc[:3]), "shape")
    _expect_bad(pa, lambda: pa.make_cache(kc, kc.to(torch.uint8)), "dtype")
    _expect_bad(pa, lambda: pa.make_cache(kc, kc), "GPU tensor")
    _expect_bad(pa, lambda: pa.make_cache(kc.transpose(2, 3).contiguous().transpose(2, 3), kc),
                "contiguous")
    c8 = torch.zeros((4, 2, 16, 64), dtype=torch.uint8)
    with pytest.raises(pa.PagedAttnError):
        pa.make_cache(c8, c8)  # E4M3 without scales
    _expect_bad(pa, lambda: pa.make_cache(c8, c8, torch.ones(4, 3), torch.ones(4, 2)), "shape")
    _expect_bad(pa, lambda: pa.make_cache(c8, c8, torch.ones(4, 2, dtype=torch.float64),
                                          torch.ones(4, 2)), "dtype")
    _expect_bad(pa, lambda: pa.make_cache(kc, kc, torch.ones(4, 2), torch.ones(4, 2)), "no scales")
    # a descriptor for the calls below (raw fields: never dereferenced)
    c = cache(pa, num_blocks=4, num_kv_heads=2, block_size=16, head_dim=64)
    k_new = torch.zeros((3, 2, 64), dtype=bf)
    slots = torch.zeros(3, dtype=i64)
    _expect_bad(pa, lambda: pa.kv_append(c, k_new, k_new, slots.to(i32)), "dtype")
    _expect_bad(pa, lambda: pa.kv_append(c, k_new, k_new, torch.zeros(4, dtype=i64)), "shape")
    _expect_bad(pa, lambda: pa.kv_append(c, k_new[:, :1], k_new, slots), "shape")
    _expect_bad(pa, lambda: pa.kv_append(c, k_new, k_new.float(), slots), "dtype")
    _expect_bad(pa, lambda: pa.kv_append(c, k_new, k_new, slots), "GPU tensor")
    # forward: q rows must equal sum(incr); out/lse shapes follow q; tables int32 with a row
    # per sequence
    q = torch.zeros((5, 8, 64), dtype=bf)
    out = torch.zeros_like(q)
    bt = torch.zeros((2, 4), dtype=i32)
    ws = torch.zeros(256, dtype=torch.uint8)
    call = lambda **kw: pa.paged_attn_forward(**{**dict(q=q, cache=c, block_tables=bt,
                                                        hist_lens=[10, 3], incr_lens=[4, 1],
                                                        scale=0.125, out=out, workspace=ws), **kw})
    _expect_bad(pa, lambda: call(incr_lens=[4, 2]), "shape")
    _expect_bad(pa, lambda: call(hist_lens=[10]), "equal length")
    _expect_bad(pa, lambda: call(q=q.float()), "dtype")
    _expect_bad(pa, lambda: call(q=torch.zeros((5, 8, 128), dtype=bf)), "shape")
    _expect_bad(pa, lambda: call(out=torch.zeros((5, 4, 64), dtype=bf)), "shape")
    _expect_bad(pa, lambda: call(lse_out=torch.zeros((5, 8), dtype=torch.float64)), "dtype")
    _expect_bad(pa, lambda: call(block_tables=bt.to(i64)), "dtype")
    _expect_bad(pa, lambda: call(block_tables=bt[:1]), "rows")
    _expect_bad(pa, lambda: call(block_tables=bt.t()), "contiguous")
    _expect_bad(pa, lambda: call(workspace=None), "workspace")
    _expect_bad(pa, lambda: call(), "GPU tensor")
    _expect_bad(pa, lambda: pa.pa_debug_gather(c, torch.zeros(2, dtype=i32), 40,
                                               torch.zeros((40, 2, 64), dtype=bf),
                                               torch.zeros((40, 2, 64), dtype=bf)), "covers")
    _expect_bad(pa, lambda: pa.pa_debug_gather(c, torch.zeros(4, dtype=i32), 40,
                                               torch.zeros((40, 2, 32), dtype=bf),
                                               torch.zeros((40, 2, 64), dtype=bf)), "shape")


def test_noalloc_rejects_steps_beyond_its_scratch(palib):
    """The no-allocation entry point refuses, before touching the device, a
    step whose plan needs more than its static scratch."""
    pa = palib
    c = cache(pa, num_blocks=1 << 30)
    h = np.full(512, 1_000_000, np.int32)  # 512 decodes over a million tokens each
    n = np.full(512, 1, np.int32)
    need = pa.pa_workspace_size(h, n, 32, c)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    st = pa.lib.paged_attn_forward_noalloc(FAKE, C.byref(c), FAKE, 62_501, h.ctypes.data_as(C.c_void_p),
                                           n.ctypes.data_as(C.c_void_p), 512, 32, 0.088, FAKE, None, None)
    assert st == pa.PA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in pa.pa_last_error()


def test_mxfp4_cache_checks(palib):
    """MXFP4 descriptors: head_dim 128 only, both scale arrays required; the
    binding tells MXFP4 from E4M3 by the scales' dtype and shape."""
    import torch
    pa = palib
    mx = pa.PA_KV_MXFP4
    assert pa.lib.kv_append(C.byref(cache(pa, dtype=mx, k_scale=FAKE, v_scale=FAKE, head_dim=64)),
                            FAKE, FAKE, FAKE, 3, None) == pa.PA_ERR_UNSUPPORTED
    assert pa.lib.kv_append(C.byref(cache(pa, dtype=mx, k_scale=None, v_scale=FAKE)),
                            FAKE, FAKE, FAKE, 3, None) == pa.PA_ERR_NULL_ARG
    assert pa.lib.kv_append(C.byref(cache(pa, dtype=mx, k_scale=FAKE, v_scale=FAKE)),
                            None, None, None, 0, None) == pa.PA_OK
    assert pa.lib.kv_append(C.byref(cache(pa, dtype=3, k_scale=FAKE, v_scale=FAKE)),
                            FAKE, FAKE, FAKE, 3, None) == pa.PA_ERR_UNSUPPORTED
    codes = torch.zeros((4, 2, 16, 64), dtype=torch.uint8)   # head_dim 128, two codes a byte
    sc = torch.zeros((4, 2, 4, 16), dtype=torch.uint8)       # [nb][hkv][d/32][bs]
    _expect_bad(pa, lambda: pa.make_cache(codes, codes, sc, sc[:, :, :3]), "shape")
    _expect_bad(pa, lambda: pa.make_cache(codes, codes, sc, torch.zeros((4, 2, 4, 16), dtype=torch.int8)), "dtype")
    _expect_bad(pa, lambda: pa.make_cache(codes, codes, sc.transpose(2, 3).contiguous(), sc), "shape")
    _expect_bad(pa, lambda: pa.make_cache(codes, codes, sc, sc), "GPU tensor")
    # the planner sizes an MXFP4 step like a bf16 one (same tiles and partials)
    hist, incr = np.array([5000, 100], np.int32), np.array([700, 1], np.int32)
    bf = pa.pa_workspace_size(hist, incr, 32, cache(pa))
    f4 = pa.pa_workspace_size(hist, incr, 32, cache(pa, dtype=mx, k_scale=FAKE, v_scale=FAKE))
    assert bf == f4 > 0


def test_step_sizes_every_format_at_head_dim_128(palib):
    """paged_attn_step's size query: bf16, E4M3 and MXFP4 caches at head_dim
    128 are sized (the same tiles and partials); head_dim 64 is rejected."""
    pa = palib
    hist, incr = np.array([5000, 100], np.int32), np.array([700, 1], np.int32)

    def size(c):
        n = C.c_size_t(0)
        st = pa.lib.paged_attn_step(C.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, 512,
                                    hist.ctypes.data_as(C.c_void_p), incr.ctypes.data_as(C.c_void_p), 2, 32,
                                    0.088, FAKE, None, None, C.byref(n), None)
        return st, n.value

    st, bf = size(cache(pa))
    assert st == pa.PA_OK and bf > 0
    for dt in (pa.PA_KV_FP8_E4M3, pa.PA_KV_MXFP4):
        st, n = size(cache(pa, dtype=dt, k_scale=FAKE, v_scale=FAKE))
        assert st == pa.PA_OK and n == bf, (dt, st, n, pa.pa_last_error())
    st, _ = size(cache(pa, head_dim=64))
    assert st == pa.PA_ERR_UNSUPPORTED
