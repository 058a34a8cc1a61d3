"""The seeded generators reproduce the workload shapes the pages print
(tests/golden/page_workload_facts.txt, one citation per line) and are
deterministic."""
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_workload_facts.txt")


def facts():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = int(v)
    return out


def test_incremental_prefill_shape_matches_page():
    f = facts()
    s = W.incremental()
    assert s.hist == [f["session_ctx_before"]]
    assert s.hist[0] + s.incr[0] == f["session_ctx_after"]
    assert W.initial().hist == [f["initial_prefill_hist"]]


def test_decode_batch_statistics():
    f = facts()
    s = W.decode_batch()
    ctx = np.array(s.hist) + 1
    assert len(ctx) == 64 and ctx.min() >= 10_000 and ctx.max() <= 262_144
    # median of 64 lognormal draws lies within +-20% of the page's median
    assert 0.8 * f["median_input"] < np.median(ctx) < 1.2 * f["median_input"]
    assert s.incr == [1] * 64


def test_mixed_step_structure():
    f = facts()
    s = W.mixed()
    assert len(s.hist) == 52 and sum(s.incr) <= 8192
    assert s.shared_prefix_tokens == f["subagent_start"]
    sub_ctx = np.array(s.hist[4:12]) + 1
    assert sub_ctx.min() >= f["subagent_start"] + 20_000 and sub_ctx.max() <= f["subagent_start"] + 50_000
    assert f["subagent_end_a"] >= 29_000 and f["subagent_end_b"] <= 60_000  # the suffix range covers both


def test_long_context_reaches_1m():
    f = facts()
    s = W.long_context()
    assert s.hist[0] + s.incr[0] == f["max_context"]


def test_generators_are_deterministic():
    a, b = W.make_batch(W.tiny()), W.make_batch(W.tiny())
    assert np.array_equal(a.block_tables, b.block_tables)
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_new, b.v_new)]:
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert sorted(a.block_tables[0].tolist()) == list(range(18))


def test_poisoning_of_unused_slots():
    b = W.make_batch(W.Spec("p", 9, 8, 2, 32, 16, [40], [9]))
    k = b.k_pool.view(torch.int16)
    bt = b.block_tables[0]
    # history tokens 0..39 finite; slots 40.. (new tokens, tail) and spare blocks NaN
    assert torch.isfinite(b.k_pool[bt[0]]).all() and torch.isfinite(b.k_pool[bt[1]]).all()
    assert torch.isfinite(b.k_pool[bt[2], :, :8]).all()
    assert torch.isnan(b.k_pool[bt[2], :, 8:]).all()
    assert torch.isnan(b.k_pool[bt[3]]).all()
    spare = sorted(set(range(b.num_blocks)) - set(bt[:4].tolist()))
    assert len(spare) >= 1 and torch.isnan(b.k_pool[spare]).all()
