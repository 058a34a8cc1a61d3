"""Shared-prefix cascade decode (paged_attn_forward_cascade) against the
fp64 oracle: sequences that share the first blocks of their block tables
read that prefix once, as one tile of all members' rows, and merge it with
their own suffix by LSE.  Cases: a small group with a non-member decode and
a prefill in the same step, groups wider than one tile (member runs), GQA
group 8, block size 64, groups the cascade does not apply to, and the mixed
step's eight sub-agents at full size; needles in the shared prefix and in
the suffixes."""
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


def cascade_step(palib, b, group_of, group_len, host):
    spec = b.spec
    c = palib.make_cache(*gpu_caches(b, host))
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    bt = torch.from_numpy(b.block_tables).to(DEV)
    need = palib.cascade_workspace_size(b.hist, b.incr, spec.num_q_heads, c, bt, group_of, group_len,
                                        spec.scale)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.full((spec.total_q, spec.num_q_heads, spec.head_dim), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    lse = torch.full((spec.total_q, spec.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    palib.paged_attn_forward_cascade(b.q, c, bt, b.hist, b.incr, spec.scale, out, ws, group_of, group_len,
                                     lse_out=lse)
    torch.cuda.synchronize()
    return out, lse, c


def check(palib, spec, group_of, group_len, what, compare_plain=True):
    nd = [(s, 0) for s in range(spec.num_seqs) if spec.hist[s] > 0 and spec.incr[s] > 0]
    spec = W.with_needles(spec, needles=nd)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    out, lse, c = cascade_step(palib, b, group_of, group_len, host)
    ref, ref_lse, after = oracle_step(b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    assert_parity(out, ref, spec.kv_dtype == "e4m3", what, needles=[(r, h) for r, h, _, _ in b.needles])
    assert_lse(lse, ref_lse, lse_bounds(b, after), what)
    if compare_plain:
        # the plain entry point on the same cache (the step's tokens already
        # appended): equal within rounding -- the key ranges differ
        plain, _ = forward(palib, b, c)
        torch.cuda.synchronize()
        d = (plain.float() - out.float()).abs().max().item()
        print(f"[cascade] {what}: max |cascade - plain| = {d:.3e}", flush=True)
        assert d <= 2e-2


def _spec(hist, incr, shared, members, hq=32, hkv=8, bs=16, cfg=80):
    return W.Spec("cascade", cfg, hq, hkv, 128, bs, hist, incr, shared_prefix_tokens=shared,
                  shared_seqs=members)


def test_cascade_small_group_in_a_mixed_step(palib):
    print("[case] cascade: 8 members over 1,024 shared tokens, a non-member decode, a prefill", flush=True)
    hist = [3000, 2500, 4100, 1500, 1100, 6000, 1300, 2000, 5000, 700]
    incr = [1, 1, 1, 1, 1, 1, 1, 5, 1, 90]  # member 7 has 5 new tokens: not in the cascade
    spec = _spec(hist, incr, 1024, list(range(8)))
    group_of = [0] * 8 + [-1, -1]
    check(palib, spec, group_of, [1024], "cascade small")


def test_cascade_member_runs_gqa8_and_block64(palib):
    print("[case] cascade: 20 members (two tiles), G 8, block 64", flush=True)
    rng = np.random.default_rng(5)
    hist = [int(x) for x in rng.integers(2100, 9000, size=20)]
    spec = _spec(hist, [1] * 20, 2048, list(range(20)), cfg=81)
    check(palib, spec, [0] * 20, [2048], "cascade 20 members")
    spec = _spec(hist[:10], [1] * 10, 2048, list(range(10)), hq=64, hkv=8, cfg=82)
    check(palib, spec, [0] * 10, [2048], "cascade G8")
    spec = _spec(hist[:6], [1] * 6, 2048, list(range(6)), bs=64, cfg=83)
    check(palib, spec, [0] * 6, [2048], "cascade block 64")


def test_cascade_declared_but_not_applicable(palib):
    """A group of one eligible member, a group of length 0 and a member whose
    history is shorter than the group's prefix run on the plain path."""
    print("[case] cascade: groups it does not apply to", flush=True)
    spec = _spec([3000, 2000, 900], [1, 1, 1], 1024, [0, 1], cfg=84)
    check(palib, spec, [0, 1, -1], [1024, 0], "cascade n/a")


def test_cascade_rejects_bad_groups(palib):
    spec = _spec([300, 300], [1, 1], 256, [0, 1], cfg=85)
    b = W.make_batch(spec, DEV)
    c = palib.make_cache(b.k_pool, b.v_pool)
    bt = torch.from_numpy(b.block_tables).to(DEV)
    for go, gl in (([0, 3], [256]), ([0, 0], [250]), ([0, -2], [256])):
        with pytest.raises(palib.PagedAttnError):
            palib.cascade_workspace_size(b.hist, b.incr, 32, c, bt, go, gl, spec.scale)


def test_cascade_mixed_step_full_size(palib):
    """The mixed step at full size: its eight sub-agents declared as one group
    over their 10,000 shared tokens; sampled sub-agent and other rows."""
    from tests.test_gpu_fullsize import compact_subset, oracle_on_subset
    spec = W.mixed()
    seqs = [0, 4, 5, 8, 11, 12, 51]
    spec = W.with_needles(spec, needles=[(s, 0) for s in (4, 5, 8, 11, 12, 51)])
    print("[case] cascade: mixed step, 8 sub-agents over 10,000 shared tokens", flush=True)
    b = W.make_batch(spec, DEV)
    group_of = [0 if s in spec.shared_seqs else -1 for s in range(spec.num_seqs)]
    out, _, _ = cascade_step(palib, b, group_of, [spec.shared_prefix_tokens], host=None)
    sub = compact_subset(b, seqs)
    n0 = spec.incr[0]
    local = [0, n0 - 1] + list(range(n0, n0 + 6))
    ref, _ = oracle_on_subset(sub, spec, local)
    grows = [int(sub["rows"][i]) for i in local]
    at = {r: i for i, r in enumerate(grows)}
    assert_parity(out[torch.as_tensor(grows, device=DEV)], ref, False, "cascade mixed",
                  needles=[(at[r], h) for r, h, _, _ in b.needles if r in at])
