"""Pins for the oracle's attention, gather, merge and kv_append (CPU only).

Nothing here re-types the oracle's formula: each test checks a consequence the
pages or the mathematics fix independently -- a 50-digit brute force at the
tiny workload's size, closed forms (constant values, identical keys, zero
scale, one dominant key, a single key), the incremental/initial/decode
relations the pages state ("ICML'26 | AMPD ..." §1 and §3: incremental
prefill reads history plus increment, initial prefill is l_hist = 0, decode
adds one token), the inclusive causal boundary, the GQA grouping, invariance
under physical placement and prefix sharing ("vLLM/V1 推理调度器": requests
hold lists of block ids, blocks are shared by reference count), and the
LSE-weighted merge of partial results ("vLLM Agentic 推理｜面向 Agent 负载的推理优化"
§4.3.3).
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.helpers import bf16_bits_of, bf16_values, bits16, host_caches, oracle_step


# ---------------------------------------------------------------------------
def test_block_count_by_enumeration():
    """cdiv(ctx, bs) equals the number of distinct blocks the tokens 0..ctx-1 touch."""
    for bs in (16, 64):
        for ctx in [0, 1, bs - 1, bs, bs + 1, 7 * bs, 7 * bs + 1, 45_700, 48_400, 1_048_576]:
            touched = len({p // bs for p in range(ctx)}) if ctx < 100_000 else (
                (ctx - 1) // bs + 1)
            assert oracle.num_blocks(ctx, bs) == touched, (ctx, bs)
    assert oracle.num_blocks(48_400, 16) == 3025
    assert oracle.num_blocks(45_700, 16) == 2857
    assert oracle.num_blocks(1_048_832, 64) == 16_388


# ---------------------------------------------------------------------------
def manual_case(K, V, Q, hist, bs=4, seed=0, spare=3):
    """Place logical K/V [ctx, hkv, d] into a permuted pool; return oracle args."""
    ctx, hkv, d = K.shape
    nblk = -(-ctx // bs)
    pool = nblk + spare
    perm = np.random.default_rng(seed).permutation(pool).astype(np.int32)
    bt = perm[:nblk][None, :].copy()
    kc = np.full((pool, hkv, bs, d), 0x7FC0, dtype=np.uint16)
    vc = kc.copy()
    kb, vb = bf16_bits_of(K), bf16_bits_of(V)
    for p in range(ctx):
        kc[bt[0, p // bs], :, p % bs, :] = kb[p]
        vc[bt[0, p // bs], :, p % bs, :] = vb[p]
    qb = bf16_bits_of(Q)
    incr = Q.shape[0]
    assert hist + incr == ctx
    return qb, kc, vc, bt, np.array([hist], np.int32), np.array([incr], np.int32)


def run_manual(K, V, Q, hist, scale, **kw):
    qb, kc, vc, bt, h, n = manual_case(K, V, Q, hist, **kw)
    return oracle.attention(qb, kc, vc, None, None, oracle.KV_BF16, bt, h, n, Q.shape[1], scale)


def test_tiny_against_50_digit_brute_force():
    """The tiny workload (1 session, 4 q / 1 KV head, d 64, 256 + 32 tokens,
    permuted 18-block table) against exact dot products and 50-digit exp/log."""
    b = W.make_batch(W.tiny())
    rows = [0, 1, 15, 16, 31]
    out, lse, (kc, vc, _, _, _) = oracle_step(b, rows=rows)
    K = bf16_values(oracle.gather(kc, b.block_tables[0], 288))[:, 0, :]
    V = bf16_values(oracle.gather(vc, b.block_tables[0], 288))[:, 0, :]
    Q = bf16_values(bits16(b.q))
    scale = Fraction(float(np.float32(b.spec.scale)))
    mpmath.mp.dps = 50
    worst = 0.0
    for i, r in enumerate(rows):
        pos = 256 + r
        for h in range(4):
            logits = [scale * sum(Fraction(float(Q[r, h, e])) * Fraction(float(K[j, e]))
                                  for e in range(64)) for j in range(pos + 1)]
            ml = [mpmath.mpf(l.numerator) / l.denominator for l in logits]
            m = max(ml)
            w = [mpmath.exp(x - m) for x in ml]
            Z = mpmath.fsum(w)
            for e in range(0, 64, 7):
                o = mpmath.fsum(w[j] * V[j, e] for j in range(pos + 1)) / Z
                worst = max(worst, abs(float(o) - out[i, h, e]))
            assert abs(float(m + mpmath.log(Z)) - lse[i, h]) < 1e-13
    assert worst < 1e-14, worst


def test_closed_form_constant_values():
    rng = np.random.default_rng(1)
    ctx, d = 37, 16
    K = rng.standard_normal((ctx, 1, d))
    c = rng.standard_normal(d)
    V = np.broadcast_to(c, (ctx, 1, d)).copy()
    Q = rng.standard_normal((9, 2, d))
    out, _ = run_manual(K, V, Q, ctx - 9, 0.25)
    cb = bf16_values(bf16_bits_of(c))
    assert np.max(np.abs(out - cb)) < 1e-14


def test_closed_form_identical_keys_and_zero_scale_give_causal_mean():
    rng = np.random.default_rng(2)
    ctx, d, n = 29, 8, 6
    V = rng.standard_normal((ctx, 1, d))
    Vb = bf16_values(bf16_bits_of(V))[:, 0, :]
    Q = rng.standard_normal((n, 3, d))
    Ksame = np.broadcast_to(rng.standard_normal(d), (ctx, 1, d)).copy()
    for K, scale in [(Ksame, 0.3), (rng.standard_normal((ctx, 1, d)), 0.0)]:
        out, lse = run_manual(K, V, Q, ctx - n, scale)
        for i in range(n):
            pos = ctx - n + i
            mean = [float(sum(Fraction(float(x)) for x in Vb[:pos + 1, e]) / (pos + 1))
                    for e in range(d)]
            assert np.max(np.abs(out[i] - np.array(mean)[None, :])) < 1e-14
        if scale == 0.0:  # lse = ln(#keys)
            assert np.allclose(lse, np.log(np.arange(ctx - n, ctx) + 1)[:, None], atol=1e-14)


def test_closed_form_one_dominant_key():
    d, ctx = 8, 20
    rng = np.random.default_rng(3)
    K = np.zeros((ctx, 1, d))
    K[11, 0, 0] = 320.0                      # logit 0.125 * 320 = 40 for a one-hot query
    V = rng.standard_normal((ctx, 1, d))
    Vb = bf16_values(bf16_bits_of(V))[:, 0, :]
    Q = np.zeros((1, 1, d))
    Q[0, 0, 0] = 1.0
    out, lse = run_manual(K, V, Q, ctx - 1, 0.125)
    e40 = np.exp(40.0)
    ref = (e40 * Vb[11] + (Vb.sum(0) - Vb[11])) / (e40 + ctx - 1)
    assert np.max(np.abs(out[0, 0] - ref)) < 1e-15
    assert abs(lse[0, 0] - (40.0 + np.log1p((ctx - 1) / e40))) < 1e-13


def test_single_key_returns_its_value():
    rng = np.random.default_rng(4)
    K, V, Q = rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 4, 8))
    out, lse = run_manual(K, V, Q, 0, 0.35)
    Vb = bf16_values(bf16_bits_of(V))[0, 0]
    assert np.array_equal(out[0], np.broadcast_to(Vb, (4, 8)))


def test_causal_boundary_is_inclusive():
    """Row at position p ignores keys > p and depends on key p itself."""
    rng = np.random.default_rng(5)
    ctx, d, n = 24, 8, 5
    K, V, Q = rng.standard_normal((ctx, 1, d)), rng.standard_normal((ctx, 1, d)), rng.standard_normal((n, 1, d))
    base, _ = run_manual(K, V, Q, ctx - n, 0.3)
    for i in range(n):
        p = ctx - n + i
        K2, V2 = K.copy(), V.copy()
        K2[p + 1:] += 5.0
        V2[p + 1:] -= 3.0
        o2, _ = run_manual(K2, V2, Q, ctx - n, 0.3)
        assert np.array_equal(o2[i], base[i])
        V3 = V.copy()
        V3[p] += 4.0
        o3, _ = run_manual(K, V3, Q, ctx - n, 0.3)
        assert np.max(np.abs(o3[i] - base[i])) > 1e-3


def test_gqa_grouping_contiguous():
    """Query head h reads KV head h // (Hq / Hkv): perturbing KV head k moves
    exactly the heads of group k."""
    rng = np.random.default_rng(6)
    ctx, d, hkv, hq = 12, 8, 2, 6
    K, V = rng.standard_normal((ctx, hkv, d)), rng.standard_normal((ctx, hkv, d))
    Q = rng.standard_normal((3, hq, d))
    base, _ = run_manual(K, V, Q, ctx - 3, 0.3)
    for k in range(hkv):
        V2 = V.copy()
        V2[:, k] += 2.0
        o2, _ = run_manual(K, V2, Q, ctx - 3, 0.3)
        moved = [h for h in range(hq) if not np.array_equal(o2[:, h], base[:, h])]
        assert moved == list(range(3 * k, 3 * k + 3))


# ---------------------------------------------------------------------------
def _small_spec(hist, incr, **kw):
    return W.Spec("small", 9, 8, 2, 32, 16, hist, incr, **kw)


def test_incremental_equals_tail_of_initial_prefill():
    """Incremental prefill over [hist | incr] = last incr rows of the initial
    prefill (hist = 0) of the concatenated sequence."""
    hist, incr = 77, 21
    b_inc = W.make_batch(_small_spec([hist], [incr]))
    out_inc, lse_inc, (kc, vc, _, _, _) = oracle_step(b_inc)
    # full prefill of the same content: all 98 tokens are queries
    K = oracle.gather(kc, b_inc.block_tables[0], hist + incr)
    V = oracle.gather(vc, b_inc.block_tables[0], hist + incr)
    rng = np.random.default_rng(0)
    Qfull = bits16(W.randn_bf16((hist + incr, 8, 32), "cpu", 123))
    Qfull[hist:] = bits16(b_inc.q)
    bt = b_inc.block_tables
    out_full, lse_full = oracle.attention(Qfull, kc, vc, None, None, oracle.KV_BF16, bt,
                                          np.array([0], np.int32), np.array([hist + incr], np.int32),
                                          8, b_inc.spec.scale)
    assert np.array_equal(out_full[hist:], out_inc)
    assert np.array_equal(lse_full[hist:], lse_inc)
    # decode = last row: hist' = ctx - 1, incr' = 1, same q
    out_dec, lse_dec = oracle.attention(Qfull[-1:], kc, vc, None, None, oracle.KV_BF16, bt,
                                        np.array([hist + incr - 1], np.int32),
                                        np.array([1], np.int32), 8, b_inc.spec.scale)
    assert np.array_equal(out_dec[0], out_full[-1])


def test_tiny_decode_equals_last_prefill_row():
    b = W.make_batch(W.tiny())
    out, _, (kc, vc, _, _, _) = oracle_step(b)
    q_last = bits16(b.q)[31:32]
    out_dec, _ = oracle.attention(q_last, kc, vc, None, None, oracle.KV_BF16, b.block_tables,
                                  np.array([287], np.int32), np.array([1], np.int32), 4, b.spec.scale)
    assert np.array_equal(out_dec[0], out[31])


def test_probabilities_sum_to_one():
    b = W.make_batch(_small_spec([150, 40], [3, 17]))
    _, _, (kc, vc, _, _, _) = oracle_step(b)
    q = bits16(b.q)
    for r, (s, pos) in enumerate([(0, 150), (0, 152), (1, 40), (1, 56)]):
        row = r if s == 0 else 3 + (pos - 40)
        _, _, probs = oracle.attention_partial(q[row, 5], kc, vc, None, None, 0,
                                               b.block_tables[s], 5 // 4, pos, 0, pos + 1,
                                               b.spec.scale, want_probs=True)
        assert len(probs) == pos + 1 and np.all(probs > 0)
        assert abs(probs.sum() - 1.0) <= 1e-12


def test_invariant_under_physical_permutation():
    s1 = _small_spec([300, 61, 0], [5, 1, 40], perm_seed=0)
    s2 = _small_spec([300, 61, 0], [5, 1, 40], perm_seed=7)
    b1, b2 = W.make_batch(s1), W.make_batch(s2)
    assert not np.array_equal(b1.block_tables, b2.block_tables)
    o1, l1, _ = oracle_step(b1)
    o2, l2, _ = oracle_step(b2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_shared_prefix_equals_unshared_copies():
    """Sub-agents reading one physical copy of a prefix = each holding its own copy."""
    spec = _small_spec([100, 90, 130], [1, 1, 4], shared_prefix_tokens=64, shared_seqs=[0, 1, 2])
    b = W.make_batch(spec)
    assert (b.block_tables[:, :4] == b.block_tables[0, :4]).all()
    out_sh, lse_sh, (kc, vc, _, _, _) = oracle_step(b)
    # unshare: copy the 4 prefix blocks for seqs 1 and 2 into fresh pool blocks
    nb = kc.shape[0]
    kc2 = np.concatenate([kc, kc[b.block_tables[0, :4]], kc[b.block_tables[0, :4]]])
    vc2 = np.concatenate([vc, vc[b.block_tables[0, :4]], vc[b.block_tables[0, :4]]])
    bt2 = b.block_tables.copy()
    bt2[1, :4] = np.arange(nb, nb + 4)
    bt2[2, :4] = np.arange(nb + 4, nb + 8)
    out_un, lse_un = oracle.attention(bits16(b.q), kc2, vc2, None, None, 0, bt2, b.hist, b.incr, 8,
                                      spec.scale)
    assert np.array_equal(out_sh, out_un) and np.array_equal(lse_sh, lse_un)


def test_lse_merge_of_random_partitions_equals_whole():
    b = W.make_batch(_small_spec([500], [9]))
    _, _, (kc, vc, _, _, _) = oracle_step(b)
    q = bits16(b.q)
    rng = np.random.default_rng(9)
    for trial in range(12):
        row, h = int(rng.integers(0, 9)), int(rng.integers(0, 8))
        pos = 500 + row
        o_all, lse_all = oracle.attention_partial(q[row, h], kc, vc, None, None, 0,
                                                  b.block_tables[0], h // 4, pos, 0, pos + 1,
                                                  b.spec.scale)
        n_parts = int(rng.integers(1, 9))
        cuts = np.sort(rng.integers(0, pos + 40, size=n_parts - 1))  # may exceed pos: empty parts
        edges = [0] + cuts.tolist() + [pos + 40]
        parts = [oracle.attention_partial(q[row, h], kc, vc, None, None, 0, b.block_tables[0],
                                          h // 4, pos, lo, hi, b.spec.scale)
                 for lo, hi in zip(edges[:-1], edges[1:])]
        o, lse = oracle.merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
        assert np.max(np.abs(o - o_all)) <= 1e-12 * max(1.0, np.max(np.abs(o_all)))
        assert abs(lse - lse_all) <= 1e-12 * max(1.0, abs(lse_all))
    # all parts empty
    o, lse = oracle.merge(np.zeros((2, 4)), np.array([-np.inf, -np.inf]))
    assert lse == -np.inf and not np.any(o)


def test_output_magnitude_statistics():
    """With N(0,1) q/k/v and scale 1/sqrt(d) the logits are ~N(0,1), so each
    output coordinate has standard deviation about sqrt(e / n) over n keys."""
    b = W.make_batch(_small_spec([4000], [8]))
    out, _, _ = oracle_step(b)
    ratio = out.std() / np.sqrt(np.e / 4004)
    assert 0.75 < ratio < 1.3, ratio


# ---------------------------------------------------------------------------
def test_kv_append_bf16_writes_only_named_slots():
    b = W.make_batch(_small_spec([40, 0, 17], [9, 12, 1]))
    kc, vc, _, _, dt = host_caches(b)
    k0, v0 = kc.copy(), vc.copy()
    slots = b.slot_mapping.numpy().copy()
    slots[3] = -1  # skipped token
    oracle.kv_append(kc, vc, None, None, dt, bits16(b.k_new), bits16(b.v_new), slots)
    bs = 16
    written = np.zeros(kc.shape[:1] + (kc.shape[2],), bool)  # [nb, bs]
    kn, vn = bits16(b.k_new), bits16(b.v_new)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        written[s // bs, s % bs] = True
        assert np.array_equal(kc[s // bs, :, s % bs, :], kn[t])
        assert np.array_equal(vc[s // bs, :, s % bs, :], vn[t])
    mask = ~written[:, None, :, None] & np.ones(kc.shape, bool)
    assert np.array_equal(kc[mask], k0[mask]) and np.array_equal(vc[mask], v0[mask])
    s3 = b.slot_mapping[3].item()
    assert np.all(kc[s3 // bs, :, s3 % bs, :] == 0x7FC0)  # still the NaN poison


def test_kv_append_e4m3_matches_torch_cast():
    spec = W.Spec("small8", 9, 8, 2, 32, 64, [100], [60], kv_dtype="e4m3")
    b = W.make_batch(spec)
    kc, vc, ks, vs, dt = host_caches(b)
    oracle.kv_append(kc, vc, ks, vs, dt, bits16(b.k_new), bits16(b.v_new), b.slot_mapping.numpy())
    slots = b.slot_mapping.numpy()
    blk, off = slots // 64, slots % 64
    ref_k = (b.k_new.float() / b.k_scale[torch.from_numpy(blk)][:, :, None]).to(torch.float8_e4m3fn)
    ref_v = (b.v_new.float() / b.v_scale[torch.from_numpy(blk)][:, :, None]).to(torch.float8_e4m3fn)
    assert np.array_equal(kc[blk, :, off, :], ref_k.view(torch.uint8).numpy())
    assert np.array_equal(vc[blk, :, off, :], ref_v.view(torch.uint8).numpy())


def test_gather_identity_table_is_contiguous_copy():
    rng = np.random.default_rng(8)
    pool = rng.integers(0, 65535, size=(6, 2, 4, 8), dtype=np.uint16)
    ident = np.arange(6, dtype=np.int32)
    g = oracle.gather(pool, ident, 22)
    assert np.array_equal(g, pool.transpose(0, 2, 1, 3).reshape(24, 2, 8)[:22])
