"""The parity bars can fail (CPU only): on a needled workload, an output
computed through a shifted block table, or no output at all, must be rejected
by the same check the GPU tests use, while the exact result rounded to bf16
passes.  The planted mistakes live in inputs to the oracle, on the CPU."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.helpers import bf16_bits_of, bf16_values, bits16, host_caches, lse_bounds, oracle_step
from tests.parity import REL_BF16, assert_lse, assert_parity, rel_fro


@pytest.fixture(scope="module")
def case():
    spec = W.Spec("gate", 91, 8, 2, 128, 16, [20_000, 3_000], [64, 1])
    spec = W.with_needles(spec, needles=[(0, 0), (0, 63), (0, 17), (1, 0)])
    b = W.make_batch(spec)
    host = host_caches(b)
    ref, ref_lse, after = oracle_step(b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x
                                                      for x in host))
    needles = [(r, h) for r, h, _, _ in b.needles]
    return b, ref, ref_lse, after, needles


def _bf16_round(x):
    return bf16_values(bf16_bits_of(x))


def test_exact_result_passes(case):
    b, ref, ref_lse, after, needles = case
    assert_parity(_bf16_round(ref), ref, False, "bf16(exact)", needles=needles)
    # the needled rows are dominated by their needle: |o| ~ 1
    for r, h in needles:
        assert np.linalg.norm(ref[r, h]) > 3.0


def _fails_everywhere(wrong, wrong_lse, b, ref, ref_lse, after, needles, what):
    with pytest.raises(AssertionError):
        assert_parity(_bf16_round(wrong), ref, False, what, needles=needles)
    # the relative bar alone rejects it, on the needled and on the other rows
    mask = np.zeros(ref.shape[:2], bool)
    for r, h in needles:
        mask[r, h] = True
    assert rel_fro(wrong[mask], ref[mask]) > 10 * REL_BF16
    assert rel_fro(wrong[~mask], ref[~mask]) > 10 * REL_BF16
    with pytest.raises(AssertionError):
        assert_lse(wrong_lse, ref_lse, lse_bounds(b, after), what)


def test_block_ids_off_by_one_fail(case):
    """Every block read from the physical block after the one the table names
    (the poisoned, never-written slots of this copy are filled with finite
    values, so only the addressing is wrong)."""
    b, ref, ref_lse, after, needles = case
    kc, vc, ks, vs, dt = after
    rng = np.random.default_rng(5)
    fin_k, fin_v = kc.copy(), vc.copy()
    for arr in (fin_k, fin_v):
        nan = (arr & 0x7FFF) > 0x7F80
        arr[nan] = bf16_bits_of(rng.standard_normal(int(nan.sum())).astype(np.float32))
    nb = kc.shape[0]
    bt = b.block_tables.copy()
    bt[bt >= 0] = (bt[bt >= 0] + 1) % nb
    wrong, wrong_lse = oracle.attention(bits16(b.q), fin_k, fin_v, ks, vs, dt, bt, b.hist, b.incr,
                                        b.spec.num_q_heads, b.spec.scale)
    _fails_everywhere(wrong, wrong_lse, b, ref, ref_lse, after, needles, "block ids + 1")


def test_wrong_kv_head_fails(case):
    """Every query head reads the next KV head's keys and values: wrong data
    of the same N(0, 1) distribution."""
    b, ref, ref_lse, after, needles = case
    kc, vc, ks, vs, dt = after
    kr = np.ascontiguousarray(np.roll(kc, 1, axis=1))
    vr = np.ascontiguousarray(np.roll(vc, 1, axis=1))
    wrong, wrong_lse = oracle.attention(bits16(b.q), kr, vr, ks, vs, dt, b.block_tables, b.hist,
                                        b.incr, b.spec.num_q_heads, b.spec.scale)
    _fails_everywhere(wrong, wrong_lse, b, ref, ref_lse, after, needles, "kv head + 1")


def test_zero_output_fails(case):
    b, ref, ref_lse, after, needles = case
    with pytest.raises(AssertionError):
        assert_parity(np.zeros_like(ref), ref, False, "zeros", needles=needles)
    # and without needles, where |o| is small: the relative bar still rejects it
    mask = np.ones(ref.shape[:2], bool)
    for r, h in needles:
        mask[r, h] = False
    with pytest.raises(AssertionError):
        assert_parity(np.zeros_like(ref[mask])[:, None], ref[mask][:, None], False, "zeros, plain rows")


def test_lse_bound_holds_for_bf16_rounded_probabilities(case):
    """The 384-row prefill's a-priori LSE bound covers what its roundings can
    do: l summed from probabilities each rounded to bf16 (the oracle's own
    probabilities of the prefill rows, rounded one by one) stays inside it."""
    b, ref, ref_lse, after, needles = case
    kc, vc, ks, vs, dt = after
    bound = lse_bounds(b, after)
    bt = b.block_tables[0]
    qb = bits16(b.q)
    G = b.spec.num_q_heads // b.spec.num_kv_heads
    worst = 0.0
    for r in (0, 17, 63):
        for h in (0, 5):
            pos = int(b.hist[0]) + r
            _, lse, probs = oracle.attention_partial(qb[r, h], kc, vc, ks, vs, dt, bt, h // G, pos, 0,
                                                     pos + 1, b.spec.scale, want_probs=True)
            # probabilities relative to the row's largest term, rounded to bf16
            w = probs / probs.max()
            wr = bf16_values(bf16_bits_of(w.astype(np.float32)))
            got = lse + np.log(wr.sum() / w.sum())
            err = abs(got - ref_lse[r, h])
            assert err <= bound[r, h], (r, h, err, bound[r, h])
            worst = max(worst, err / bound[r, h])
    print(f"worst err/bound {worst:.3f}")
