"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one.

The oracle sees a compact host copy of only the sampled sequences' blocks
(block ids renumbered), which is equivalent by the placement invariance the
oracle's own tests pin."""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_parity, forward, gpu_caches
from tests.helpers import bits16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def compact_subset(b, seqs):
    """Host copy of the history blocks of `seqs`, renumbered 0..n-1, plus the
    subset's lengths, tables, new-token rows and their slots."""
    bs = b.spec.block_size
    rowstart = np.concatenate([[0], np.cumsum(b.incr.astype(np.int64))])
    ids = []
    for s in seqs:
        ctx = int(b.hist[s]) + int(b.incr[s])
        ids.extend(b.block_tables[s, :-(-ctx // bs)].tolist())
    uniq = sorted(set(ids))
    remap = {p: i for i, p in enumerate(uniq)}
    sel = torch.as_tensor(uniq, dtype=torch.long, device=b.k_pool.device)
    kh = bits16(b.k_pool[sel])
    vh = bits16(b.v_pool[sel])
    maxb = max(-(-(int(b.hist[s]) + int(b.incr[s])) // bs) for s in seqs)
    bt = np.full((len(seqs), maxb), -1, np.int32)
    rows = []
    for i, s in enumerate(seqs):
        n = -(-(int(b.hist[s]) + int(b.incr[s])) // bs)
        bt[i, :n] = [remap[p] for p in b.block_tables[s, :n]]
        rows.extend(range(int(rowstart[s]), int(rowstart[s + 1])))
    rows = np.array(rows, dtype=np.int64)
    rsel = torch.as_tensor(rows, device=b.q.device)
    slots = b.slot_mapping[rsel].cpu().numpy()
    new_slots = np.array([remap[int(x) // bs] * bs + int(x) % bs for x in slots], np.int64)
    ks = vs = None
    if b.k_scale is not None:
        ks = b.k_scale[sel].cpu().numpy().astype(np.float32)
        vs = b.v_scale[sel].cpu().numpy().astype(np.float32)
    return dict(k=kh, v=vh, ks=ks, vs=vs, bt=bt, hist=b.hist[seqs], incr=b.incr[seqs], rows=rows,
                q=bits16(b.q[rsel]), k_new=bits16(b.k_new[rsel]), v_new=bits16(b.v_new[rsel]),
                slots=new_slots, sel=sel)


def oracle_on_subset(sub, spec, local_rows):
    if spec.kv_dtype == "e4m3":
        kc, vc, dt = oracle.quantize_pool(sub["k"], sub["ks"]), oracle.quantize_pool(sub["v"], sub["vs"]), oracle.KV_E4M3
    else:
        kc, vc, dt = sub["k"].copy(), sub["v"].copy(), oracle.KV_BF16
    oracle.kv_append(kc, vc, sub["ks"], sub["vs"], dt, sub["k_new"], sub["v_new"], sub["slots"])
    t = time.time()
    out, lse = oracle.attention(sub["q"], kc, vc, sub["ks"], sub["vs"], dt, sub["bt"], sub["hist"],
                                sub["incr"], spec.num_q_heads, spec.scale, rows=local_rows)
    print(f"[oracle] {len(local_rows)} rows x {spec.num_q_heads} heads in {time.time() - t:.1f}s "
          f"({oracle.num_threads()} threads)", flush=True)
    return out, (kc, vc, dt)


def gpu_full_step(palib, b, host_codes=None):
    if b.spec.kv_dtype == "e4m3":
        k = torch.from_numpy(host_codes[0]).to(DEV)
        v = torch.from_numpy(host_codes[1]).to(DEV)
        caches = (k, v, b.k_scale, b.v_scale)
    else:
        caches = gpu_caches(b)
    c = palib.make_cache(*caches)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    out, _ = forward(palib, b, c)
    torch.cuda.synchronize()
    return out, c, caches


def plan_tiles(palib, spec):
    """(first row, tokens) of every prefill tile the library's planner makes
    for this step, from its work list (pa_debug_plan): the tile height is the
    kernel's, so boundary rows are sampled where tiles really meet."""
    coded = spec.kv_dtype != "bf16"
    kind = {"bf16": palib.PA_KV_BF16, "e4m3": palib.PA_KV_FP8_E4M3, "mxfp4": palib.PA_KV_MXFP4}[spec.kv_dtype]
    c = palib.pa_kv_cache(0x1000, 0x1000, 0x1000 if coded else None, 0x1000 if coded else None, 1,
                          spec.num_kv_heads, spec.block_size, spec.head_dim, kind)
    items, counts = palib.pa_debug_plan(spec.hist, spec.incr, spec.num_q_heads, c)
    pre = items[:counts[0]]
    return sorted({(int(r), int(n)) for r, n in zip(pre[:, 2], pre[:, 4])})


def tile_boundary_rows(tiles, seq_row0, n, rng, k=8):
    """Local rows of one sequence's increment: the first and last row of its
    first, middle and last tiles and of the tiles around them, plus k random rows."""
    mine = [(r - seq_row0, t) for r, t in tiles if seq_row0 <= r < seq_row0 + n]
    rows = {0, n - 1}
    for i in sorted({0, 1, len(mine) // 2, len(mine) - 2, len(mine) - 1}):
        if 0 <= i < len(mine):
            r, t = mine[i]
            rows |= {r, r + t - 1}
    rows |= set(int(x) for x in rng.integers(0, n, size=k))
    return sorted(rows)


def local_needles(b, rows):
    """(index into `rows`, head) of the batch's needles among the sampled rows."""
    at = {r: i for i, r in enumerate(rows)}
    return [(at[r], h) for r, h, _, _ in b.needles if r in at]


PREFILL = [W.incremental(), W.initial(), W.incremental(131_072, 2_700, "incremental_128k")]


# (an initial prefill has no history to hold a needle: plain only)
@pytest.mark.parametrize("spec,needled", [(PREFILL[0], False), (PREFILL[0], True), (PREFILL[1], False),
                                          (PREFILL[2], False), (PREFILL[2], True)],
                         ids=["incremental_45.7k_to_48.4k-plain", "incremental_45.7k_to_48.4k-needles",
                              "initial_45.7k-plain", "incremental_128k-plain", "incremental_128k-needles"])
def test_single_session_prefill(palib, spec, needled):
    tiles = plan_tiles(palib, spec)
    rows = tile_boundary_rows(tiles, 0, spec.incr[0], np.random.default_rng(1))
    if needled:
        spec = W.with_needles(spec, needles=[(0, r) for r in rows[::2]])
    print(f"[case] {spec.name} hist={spec.hist} incr={spec.incr} needled={needled} "
          f"tiles={len(tiles)} rows={rows}", flush=True)
    b = W.make_batch(spec, DEV)
    sub = compact_subset(b, [0])
    out, _, _ = gpu_full_step(palib, b)
    ref, _ = oracle_on_subset(sub, spec, rows)
    assert_parity(out[rows], ref, False, spec.name, needles=local_needles(b, rows))


@pytest.mark.parametrize("needled", [False, True], ids=["plain", "needles"])
def test_decode_batch(palib, needled):
    spec = W.decode_batch()
    ctx = np.array(spec.hist) + 1
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 7, 33, 50})
    if needled:
        spec = W.with_needles(spec, needles=[(s, 0) for s in seqs])
    print(f"[case] decode_batch sessions=64 sum_ctx={sum(spec.hist) + 64} needled={needled}", flush=True)
    b = W.make_batch(spec, DEV)
    sub = compact_subset(b, seqs)
    out, _, _ = gpu_full_step(palib, b)
    ref, _ = oracle_on_subset(sub, spec, list(range(len(seqs))))
    assert_parity(out[torch.as_tensor(sub["rows"], device=DEV)], ref, False, "decode_batch",
                  needles=local_needles(b, list(sub["rows"])))


@pytest.mark.parametrize("needled", [False, True], ids=["plain", "needles"])
def test_mixed_step_with_shared_prefix(palib, needled):
    spec = W.mixed()
    seqs = [0, 3, 4, 5, 11, 12, 51]
    n0, n3 = spec.incr[0], spec.incr[3]
    tiles = plan_tiles(palib, spec)
    rs = np.random.default_rng(2)
    loc0 = tile_boundary_rows(tiles, 0, n0, rs, k=3)
    row3 = int(np.sum(spec.incr[:3]))
    loc3 = tile_boundary_rows(tiles, row3, n3, rs, k=3)
    if needled:
        spec = W.with_needles(spec, needles=[(0, loc0[0]), (0, loc0[-1]), (3, loc3[len(loc3) // 2])]
                              + [(s, 0) for s in (4, 5, 11, 12, 51)])
    print(f"[case] mixed incr={spec.incr[:4]} needled={needled}", flush=True)
    b = W.make_batch(spec, DEV)
    sub = compact_subset(b, seqs)
    out, _, _ = gpu_full_step(palib, b)
    local = loc0 + [n0 + r for r in loc3] + list(range(n0 + n3, n0 + n3 + 5))
    ref, _ = oracle_on_subset(sub, spec, local)
    grows = [int(sub["rows"][i]) for i in local]
    assert_parity(out[torch.as_tensor(grows, device=DEV)], ref, False, "mixed",
                  needles=local_needles(b, grows))


@pytest.mark.parametrize("needled", [False, True], ids=["plain", "needles"])
def test_long_context_fp8(palib, needled):
    """1M-token history in E4M3 (block 64): the incremental prefill of 4,096
    tokens, then 256 decode steps (append one token, attend); sampled rows of
    the prefill (tile boundaries from the plan) and the first and last decode
    steps are checked.  The needled variant plants needles for sampled
    prefill rows and for both checked decode steps."""
    spec = W.long_context()
    tiles = plan_tiles(palib, spec)
    rows = tile_boundary_rows(tiles, 0, spec.incr[0], np.random.default_rng(3), k=2)
    checked = {1, 256}
    if needled:
        spec = W.with_needles(spec, needles=[(0, r) for r in rows[::2]], decode_steps=sorted(checked))
    print(f"[case] long_context hist=1044480 incr=4096 e4m3 needled={needled} rows={rows}", flush=True)
    b = W.make_batch(spec, DEV)
    kh, vh = bits16(b.k_pool), bits16(b.v_pool)
    ks, vs = b.k_scale.cpu().numpy(), b.v_scale.cpu().numpy()
    codes = (oracle.quantize_pool(kh, ks), oracle.quantize_pool(vh, vs))
    del kh, vh
    out, c, caches = gpu_full_step(palib, b, codes)
    kc, vc = codes
    oracle.kv_append(kc, vc, ks, vs, oracle.KV_E4M3, bits16(b.k_new), bits16(b.v_new),
                     b.slot_mapping.cpu().numpy())
    torch.cuda.synchronize()
    # GPU cache after the quantising append equals the oracle's, byte for byte
    assert torch.equal(caches[0].cpu(), torch.from_numpy(kc))
    assert torch.equal(caches[1].cpu(), torch.from_numpy(vc))
    t = time.time()
    ref, _ = oracle.attention(bits16(b.q), kc, vc, ks, vs, oracle.KV_E4M3, b.block_tables, b.hist,
                              b.incr, 32, spec.scale, rows=rows)
    print(f"[oracle] prefill rows in {time.time() - t:.1f}s", flush=True)
    assert_parity(out[rows], ref, True, "long_context prefill", needles=local_needles(b, rows))
    # decode steps
    first = 1_048_576
    for step in range(1, 257):
        q, k1, v1 = W.decode_step_tokens(spec, step, DEV)
        pos = first + step - 1
        slot = torch.tensor([W.slot_of(b, 0, pos)], dtype=torch.int64, device=DEV)
        palib.kv_append(c, k1, v1, slot)
        outd, _ = forward(palib, b, c, q=q, hist=np.array([pos], np.int32),
                          incr=np.array([1], np.int32))
        if step in checked:
            torch.cuda.synchronize()
            oracle.kv_append(kc, vc, ks, vs, oracle.KV_E4M3, bits16(k1), bits16(v1),
                             slot.cpu().numpy())
            refd, _ = oracle.attention(bits16(q), kc, vc, ks, vs, oracle.KV_E4M3, b.block_tables,
                                       [pos], [1], 32, spec.scale)
            nd = [(0, b.decode_needles[step][0])] if step in b.decode_needles else []
            assert_parity(outd, refd, True, f"long_context decode step {step}", needles=nd)
        else:
            # keep the oracle's cache in step with the GPU's
            oracle.kv_append(kc, vc, ks, vs, oracle.KV_E4M3, bits16(k1), bits16(v1),
                             slot.cpu().numpy())
    torch.cuda.synchronize()
