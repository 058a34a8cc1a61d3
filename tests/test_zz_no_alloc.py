"""paged_attn_forward_noalloc (static scratch, for callers that cannot
allocate) against paged_attn_forward (caller's workspace) through the C ABI:
two calls in a row, the second with a smaller input; each output equals the
workspace entry point's bit for bit and meets the oracle bars."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import forward, gpu_caches
from tests.helpers import host_caches, oracle_step
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _one(palib, spec):
    b = W.make_batch(spec, DEV)
    host = host_caches(b)
    k, v, ks, vs = gpu_caches(b, host)
    c = palib.make_cache(k, v, ks, vs)
    palib.kv_append(c, b.k_new, b.v_new, b.slot_mapping)
    out_ws, _ = forward(palib, b, c)
    bt = torch.from_numpy(b.block_tables).to(DEV)
    out = torch.full_like(out_ws, float("nan"))
    lse = torch.full(out.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    palib.paged_attn_forward_noalloc(b.q, c, bt, b.hist, b.incr, spec.scale, out, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ws.view(torch.int16)), spec.name
    assert not torch.isnan(lse).any()
    ref, _, _ = oracle_step(b, caches=tuple(x.copy() if isinstance(x, np.ndarray) else x for x in host))
    assert_parity(out, ref, spec.kv_dtype == "e4m3", f"noalloc {spec.name}")


def test_noalloc_matches_workspace_entry_point(palib):
    print("[case] noalloc: prefill + split decode, then a smaller step", flush=True)
    big = W.Spec("noalloc_big", 71, 32, 8, 128, 16, [20_000, 60_000, 300], [600, 1, 40])
    small = W.Spec("noalloc_small", 72, 8, 2, 64, 16, [700], [33])
    _one(palib, big)
    _one(palib, small)
    e4 = W.Spec("noalloc_e4m3", 73, 32, 8, 128, 64, [9_000, 4_000], [200, 1], kv_dtype="e4m3")
    _one(palib, e4)
    f4 = W.Spec("noalloc_mxfp4", 74, 32, 8, 128, 16, [9_000, 4_000, 20_000], [200, 1, 1], kv_dtype="mxfp4")
    _one(palib, f4)
