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


def sample_rows(n, tile_tokens, rng, k=10):
    rows = {0, n - 1, min(n - 1, tile_tokens - 1), min(n - 1, tile_tokens)}
    rows |= set(int(x) for x in rng.integers(0, n, size=k))
    return sorted(rows)


@pytest.mark.parametrize("spec", [W.incremental(), W.initial(),
                                  W.incremental(131_072, 2_700, "incremental_128k")],
                         ids=["incremental_45.7k_to_48.4k", "initial_45.7k", "incremental_128k"])
def test_single_session_prefill(palib, spec):
    print(f"[case] {spec.name} hist={spec.hist} incr={spec.incr}", flush=True)
    b = W.make_batch(spec, DEV)
    sub = compact_subset(b, [0])
    out, _, _ = gpu_full_step(palib, b)
    rows = sample_rows(spec.incr[0], 128 // (spec.num_q_heads // spec.num_kv_heads),
                       np.random.default_rng(1))
    ref, _ = oracle_on_subset(sub, spec, rows)
    assert_parity(out[rows], ref, False, spec.name)


def test_decode_batch(palib):
    spec = W.decode_batch()
    print(f"[case] decode_batch sessions=64 sum_ctx={sum(spec.hist) + 64}", flush=True)
    b = W.make_batch(spec, DEV)
    ctx = np.array(spec.hist) + 1
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 7, 33, 50})
    sub = compact_subset(b, seqs)
    out, _, _ = gpu_full_step(palib, b)
    ref, _ = oracle_on_subset(sub, spec, list(range(len(seqs))))
    assert_parity(out[torch.as_tensor(sub["rows"], device=DEV)], ref, False, "decode_batch")


def test_mixed_step_with_shared_prefix(palib):
    spec = W.mixed()
    print(f"[case] mixed incr={spec.incr[:4]}", flush=True)
    b = W.make_batch(spec, DEV)
    seqs = [0, 3, 4, 5, 11, 12, 51]
    sub = compact_subset(b, seqs)
    out, _, _ = gpu_full_step(palib, b)
    n0, n3 = spec.incr[0], spec.incr[3]
    local = [0, n0 // 2, n0 - 1, n0, n0 + n3 - 1] + list(range(n0 + n3, n0 + n3 + 5))
    ref, _ = oracle_on_subset(sub, spec, local)
    assert_parity(out[torch.as_tensor(sub["rows"][local], device=DEV)], ref, False, "mixed")


def test_long_context_fp8(palib):
    """1M-token history in E4M3 (block 64): the incremental prefill of 4,096
    tokens, then 256 decode steps (append one token, attend); sampled rows of
    the prefill and the first and last decode steps are checked."""
    spec = W.long_context()
    print("[case] long_context hist=1044480 incr=4096 e4m3", flush=True)
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
    rows = [0, 1, 2047, 4095]
    t = time.time()
    ref, _ = oracle.attention(bits16(b.q), kc, vc, ks, vs, oracle.KV_E4M3, b.block_tables, b.hist,
                              b.incr, 32, spec.scale, rows=rows)
    print(f"[oracle] prefill rows in {time.time() - t:.1f}s", flush=True)
    assert_parity(out[rows], ref, True, "long_context prefill")
    # decode steps
    first = 1_048_576
    checked = {1, 256}
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
            assert_parity(outd, refd, True, f"long_context decode step {step}")
        else:
            # keep the oracle's cache in step with the GPU's
            oracle.kv_append(kc, vc, ks, vs, oracle.KV_E4M3, bits16(k1), bits16(v1),
                             slot.cpu().numpy())
    torch.cuda.synchronize()
