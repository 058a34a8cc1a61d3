"""GPU parity of the one-launch step (paged_attn_step: kv_append and the
attention in one persistent kernel with device-side task claiming and merges
by the last writer) against the oracle, at sizes the oracle finishes in
seconds: prefill ranges, decode items, split tiles merged in-kernel, both
block sizes, several GQA groups, bf16, E4M3 and MXFP4 KV, needles, LSE; the
cache after the step bit for bit; repeated steps on one workspace; the wait flag; and, at full
size, the mixed step against paged_attn_forward (itself checked against the
oracle at full size)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import assert_lse, assert_parity, forward, gpu_caches
from tests.helpers import bits16, bytes8, host_caches, lse_bounds, oracle_step
from tests.test_gpu_parity import _needled

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _spec(hist, incr, hq=32, hkv=8, bs=16, cfg=51, **kw):
    return W.Spec("step", cfg, hq, hkv, 128, bs, list(hist), list(incr), **kw)


def run_step_once(pa, b, caches, want_lse=True):
    spec = b.spec
    c = pa.make_cache(*caches)
    bt = torch.from_numpy(b.block_tables).to(DEV)
    need = pa.step_workspace_size(b.hist, b.incr, spec.num_q_heads, c, bt, spec.scale)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.full((spec.total_q, spec.num_q_heads, spec.head_dim), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    lse = torch.full((spec.total_q, spec.num_q_heads), float("nan"), dtype=torch.float32,
                     device=DEV) if want_lse else None
    pa.paged_attn_step(c, b.k_new, b.v_new, b.slot_mapping, b.q, bt, b.hist, b.incr, spec.scale, out, ws,
                       lse_out=lse)
    torch.cuda.synchronize()
    assert pa.pa_debug_step_flags(ws, c, b.hist, b.incr, spec.num_q_heads) == 0
    return out, lse, c, ws


CASES = {
    "mixed": _spec([5000, 900, 12_000, 0, 77, 3000], [600, 1, 1, 300, 1, 2]),
    "incremental": _spec([2000, 37], [700, 400]),
    "decode_only": _spec([100, 1000, 37, 4000, 70_000], [1, 1, 1, 1, 1]),
    "initial": _spec([0], [1000]),
    "bs64_split": _spec([60_000, 4100], [400, 1], bs=64),
    "g8": _spec([1500, 10, 640, 333], [2, 1, 2, 150], hkv=4),
    "g1": _spec([1200, 50], [300, 1], hq=8, hkv=8),
    # E4M3 and MXFP4 KV: the append quantises (MXFP4: its scale bytes too),
    # the items widen the codes
    "e4m3_mixed": _spec([5000, 900, 12_000, 0, 77, 3000], [600, 1, 1, 300, 1, 2], bs=64, kv_dtype="e4m3"),
    "e4m3_bs16_split": _spec([60_000, 4100, 333], [1, 1, 150], kv_dtype="e4m3"),
    "mxfp4_mixed": _spec([5000, 900, 12_000, 0, 77, 3000], [600, 1, 1, 300, 1, 2], kv_dtype="mxfp4"),
    "mxfp4_bs64_split": _spec([60_000, 4100, 40], [400, 1, 1], bs=64, kv_dtype="mxfp4"),
    "e4m3_g8": _spec([1500, 10, 640, 333], [2, 1, 2, 150], hkv=4, bs=64, kv_dtype="e4m3"),
    "mxfp4_g1": _spec([1200, 50], [300, 1], hq=8, hkv=8, kv_dtype="mxfp4"),
    "mxfp4_initial_and_empty": _spec([0, 700, 3000], [1000, 0, 1], bs=64, kv_dtype="mxfp4"),
    "e4m3_initial": _spec([0, 2000], [700, 1], kv_dtype="e4m3"),
}


def assert_cache_after(caches, after, kv):
    """The device cache after the step's append equals the oracle's, bit for
    bit (codes, and MXFP4's scale bytes)."""
    if kv == "bf16":
        assert np.array_equal(bits16(caches[0]), after[0]) and np.array_equal(bits16(caches[1]), after[1])
        return
    assert np.array_equal(bytes8(caches[0]), after[0]) and np.array_equal(bytes8(caches[1]), after[1])
    if kv == "mxfp4":
        assert np.array_equal(bytes8(caches[2]), after[2]) and np.array_equal(bytes8(caches[3]), after[3])


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity(palib, name):
    spec = _needled(CASES[name])
    print(f"[case] step {name}", flush=True)
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    caches = gpu_caches(b, host)
    out, lse, c, _ = run_step_once(palib, b, caches)
    ref, ref_lse, after = oracle_step(b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    # the cache after the step's append, bit for bit
    assert_cache_after(caches, after, spec.kv_dtype)
    assert_parity(out, ref, spec.kv_dtype == "e4m3", f"step {name}", needles=[(r, h) for r, h, _, _ in b.needles])
    assert_lse(lse, ref_lse, lse_bounds(b, after), f"step {name}")


def test_step_repeats_bitwise_on_one_workspace(palib):
    """Two steps on the same workspace (counters re-zeroed by the work-list
    copy) give the same bits, whatever order the work-groups claimed in."""
    spec = CASES["mixed"]
    b = W.make_batch(spec, DEV)
    caches = gpu_caches(b)
    c = palib.make_cache(*caches)
    bt = torch.from_numpy(b.block_tables).to(DEV)
    need = palib.step_workspace_size(b.hist, b.incr, spec.num_q_heads, c, bt, spec.scale)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        out = torch.empty((spec.total_q, spec.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)
        palib.paged_attn_step(c, b.k_new, b.v_new, b.slot_mapping, b.q, bt, b.hist, b.incr, spec.scale, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert palib.pa_debug_step_flags(ws, c, b.hist, b.incr, spec.num_q_heads) == 0
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_step_unsupported_formats(palib):
    spec = W.Spec("step_d64", 51, 32, 8, 64, 16, [100], [1])
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    c = palib.make_cache(*gpu_caches(b, host))
    bt = torch.from_numpy(b.block_tables).to(DEV)
    with pytest.raises(palib.PagedAttnError):
        palib.step_workspace_size(b.hist, b.incr, spec.num_q_heads, c, bt, spec.scale)


def test_mixed_step_full_size_against_forward(palib):
    """The full mixed step (4 incremental prefills, 48 decodes) through
    paged_attn_step against kv_append + paged_attn_forward on the same
    inputs: every row within the bf16 bars, and the caches equal."""
    spec = W.mixed()
    b = W.make_batch(spec, DEV)
    c1 = gpu_caches(b)
    c2 = tuple(x.clone() for x in c1 if x is not None) + (None, None)
    out1, _, _, _ = run_step_once(palib, b, c1, want_lse=False)
    cc = palib.make_cache(c2[0], c2[1])
    palib.kv_append(cc, b.k_new, b.v_new, b.slot_mapping)
    out2, _ = forward(palib, b, cc)
    torch.cuda.synchronize()
    # (bit patterns: the pools hold NaN in their unused slots)
    assert torch.equal(c1[0].view(torch.int16), c2[0].view(torch.int16))
    assert torch.equal(c1[1].view(torch.int16), c2[1].view(torch.int16))
    ref = out2.double().cpu().numpy()
    assert_parity(out1, ref, False, "mixed step: one launch against forward")


@pytest.mark.parametrize("kv", ["e4m3", "mxfp4"])
def test_long_decode_step_against_forward(palib, kv):
    """A decode step over a 1,048,575-token history (E4M3 or MXFP4 KV,
    block 64) through paged_attn_step against kv_append + paged_attn_forward
    on the same inputs: the row within the bars (needled heads within the
    relative bar too), the caches (codes and scales) equal."""
    spec = W.long_context(1_048_575, 1) if kv == "e4m3" else W.long_context_mxfp4(1_048_575, 1)
    spec = W.with_needles(spec, needles=[(0, 0)])
    print(f"[case] one-launch step, 1M-token {kv} decode", flush=True)
    b = W.make_batch(spec, DEV)
    c1 = gpu_caches(b)
    c2 = tuple(x.clone() for x in c1)
    out1, _, _, _ = run_step_once(palib, b, c1, want_lse=False)
    cc = palib.make_cache(*c2)
    palib.kv_append(cc, b.k_new, b.v_new, b.slot_mapping)
    out2, _ = forward(palib, b, cc)
    torch.cuda.synchronize()
    for x, y in zip(c1, c2):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    ref = out2.double().cpu().numpy()
    assert_parity(out1, ref, kv == "e4m3", f"one-launch {kv} decode against forward",
                  needles=[(r, h) for r, h, _, _ in b.needles])
