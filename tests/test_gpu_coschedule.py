"""The co-scheduled mixed step: a step holding prefill and decode rows
(head_dim 128; bf16, E4M3 or MXFP4 KV) whose decode items are streamed by the CUs the persistent
prefill launch leaves free and, after it, by the CUs it frees.  Which CUs run
an item does not change its arithmetic, so the decode rows equal those of
the launches run one after the other bit for bit; the prefill rows follow a
plan cut for fewer CUs and are held to the oracle bars."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import forward, gpu_caches
from tests.helpers import host_caches, lse_bounds, oracle_step
from tests.parity import assert_lse, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _forced(palib, b, c, force):
    palib.pa_debug_overlap_cus(force)
    try:
        out, lse = forward(palib, b, c, want_lse=True)
        torch.cuda.synchronize()
    finally:
        palib.pa_debug_overlap_cus(-1)
    return out, lse


def _prefill_workgroups(palib, spec, c, force):
    palib.pa_debug_overlap_cus(force)
    try:
        return len(palib.pa_debug_plan_groups(spec.hist, spec.incr, spec.num_q_heads, c)) - 1
    finally:
        palib.pa_debug_overlap_cus(-1)


@pytest.mark.parametrize("bs,kv", [(16, "bf16"), (64, "bf16"), (64, "e4m3"), (16, "mxfp4")])
def test_coscheduled_step_against_sequential_and_oracle(palib, bs, kv):
    """Two increments (one long enough to fill every CU) and six decodes (one
    split over several items), with needles: forced 0 (one launch after the
    other), 8 and 64 CUs taken from the prefill, and the planner's choice;
    decode rows bitwise equal across the modes, sampled rows of every mode
    within the bars against the oracle, and a repeated co-scheduled call
    bitwise equal to the first."""
    big = 2000
    spec = W.with_needles(
        W.Spec(f"co_{kv}_bs{bs}", 91, 32, 8, 128, bs, [20_000, 900, 5000, 7000, 200, 90_000, 4000, 12_000],
               [big, 150, 1, 1, 1, 1, 1, 1], kv_dtype=kv),
        needles=[(0, 0), (0, 95), (0, big - 1), (1, 149), (2, 0), (5, 0), (7, 0)])
    rows = sorted({0, 1, 95, 96, 191, 192, 500, 1000, 1500, big - 96, big - 1} | set(range(big, big + 156)))
    print(f"[case] co-scheduled {spec.name} hist={spec.hist} incr={spec.incr}", flush=True)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    k, v, ks, vs = gpu_caches(b, host)
    c = palib.make_cache(k, v, ks, vs)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    ref, ref_lse, after = oracle_step(
        b, rows=rows, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    bound = lse_bounds(b, after)[rows]
    at = {r: i for i, r in enumerate(rows)}
    needles = [(at[r], h) for r, h, _, _ in b.needles if r in at]
    cus = palib.pa_device_shape()[0]
    assert _prefill_workgroups(palib, spec, c, 0) == cus
    assert _prefill_workgroups(palib, spec, c, 8) == cus - 8
    assert _prefill_workgroups(palib, spec, c, 64) == cus - 64
    dec_rows = slice(big + 150, big + 156)
    outs = {}
    for force in (0, 8, 64, -1, 64):
        out, lse = _forced(palib, b, c, force)
        what = f"{spec.name} CUs taken from the prefill {force}"
        assert_parity(out[rows], ref, kv == "e4m3", what, needles=needles)
        assert_lse(lse[rows], ref_lse, bound, what)
        if force in outs:
            assert torch.equal(out.view(torch.int16), outs[force].view(torch.int16)), what
        outs[force] = out
    for force in (8, 64, -1):
        assert torch.equal(outs[force][dec_rows].view(torch.int16), outs[0][dec_rows].view(torch.int16)), force


@pytest.mark.parametrize("bs,kv", [(16, "bf16"), (64, "e4m3"), (16, "mxfp4")])
def test_small_prefill_leaves_cus_to_the_decode(palib, bs, kv):
    """A prefill too small to hold every CU: the decode items run on the CUs
    it leaves, at the same time (the planner's choice in every KV format);
    all rows against the oracle, decode rows bitwise equal to the launches
    one after the other."""
    spec = W.Spec(f"co_small_{kv}", 92, 32, 8, 128, bs, [3000, 900, 5000, 7000, 200, 40_000],
                  [300, 150, 1, 1, 1, 1], kv_dtype=kv)
    print(f"[case] co-scheduled {spec.name} hist={spec.hist} incr={spec.incr}", flush=True)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    k, v, ks, vs = gpu_caches(b, host)
    c = palib.make_cache(k, v, ks, vs)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    assert _prefill_workgroups(palib, spec, c, -1) < palib.pa_device_shape()[0]
    ref, ref_lse, after = oracle_step(
        b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    out, lse = _forced(palib, b, c, -1)
    assert_parity(out, ref, kv == "e4m3", spec.name)
    assert_lse(lse, ref_lse, lse_bounds(b, after), spec.name)
    out0, _ = _forced(palib, b, c, 0)
    assert torch.equal(out.view(torch.int16), out0.view(torch.int16))


def test_coscheduled_cascade(palib):
    """paged_attn_forward_cascade co-schedules too: the cascade items (the
    shared prefix read once for its members) and the decode items are
    claimed beside the prefill.  Sub-agents over a 4,096-token shared prefix,
    other decodes and an increment long enough to fill every CU: forced 0
    and 64 CUs and the planner's choice, every decode row bitwise equal
    across the modes, sampled rows within the bars against the oracle."""
    from tests.test_gpu_cascade import cascade_step
    big = 2000
    hist = [20_000, 9000, 7000, 12_000, 5000, 30_000, 8000, 6000]
    incr = [big, 1, 1, 1, 1, 1, 1, 1]
    members = [1, 2, 3, 4]
    spec = W.with_needles(
        W.Spec("co_cascade", 93, 32, 8, 128, 16, hist, incr, shared_prefix_tokens=4096, shared_seqs=members),
        needles=[(0, 0), (0, big - 1), (1, 0), (3, 0), (5, 0)])
    group_of = [0 if s in members else -1 for s in range(len(hist))]
    print(f"[case] co-scheduled cascade hist={hist} incr={incr} members={members}", flush=True)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    rows = sorted({0, 95, 96, 1000, big - 1} | set(range(big, big + 7)))
    ref, ref_lse, after = oracle_step(
        b, rows=rows, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    bound = lse_bounds(b, after)[rows]
    at = {r: i for i, r in enumerate(rows)}
    needles = [(at[r], h) for r, h, _, _ in b.needles if r in at]
    outs = {}
    for force in (0, 64, -1):
        palib.pa_debug_overlap_cus(force)
        try:
            out, lse, _ = cascade_step(palib, b, group_of, [4096],
                                       tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
        finally:
            palib.pa_debug_overlap_cus(-1)
        what = f"co-scheduled cascade, CUs taken from the prefill {force}"
        assert_parity(out[rows], ref, False, what, needles=needles)
        assert_lse(lse[rows], ref_lse, bound, what)
        outs[force] = out
    dec = slice(big, big + 7)
    for force in (64, -1):
        assert torch.equal(outs[force][dec].view(torch.int16), outs[0][dec].view(torch.int16)), force
