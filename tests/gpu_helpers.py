"""GPU-side test helpers: run the HIP path through the C ABI binding and
compare against the oracle.  Imported only by tests marked `gpu`."""
import numpy as np
import torch

import oracle
import workloads as W
from tests.helpers import bits16, host_caches

from tests.parity import assert_lse, assert_parity  # noqa: F401  (the bars)


def gpu_caches(batch, host=None):
    """Device caches holding the batch's history in the storage type.
    bf16: the generator's pools themselves.  e4m3: codes from the oracle's
    encoder (the caller's quantised history), uploaded; mxfp4: the oracle
    encoder's codes and scale bytes, uploaded."""
    if batch.spec.kv_dtype == "bf16":
        return batch.k_pool, batch.v_pool, None, None
    if batch.spec.kv_dtype == "mxfp4":
        kc, vc, ks, vs, _ = host if host is not None else host_caches(batch)
        dev = batch.q.device
        return tuple(torch.from_numpy(x).to(dev) for x in (kc, vc, ks, vs))
    kc, vc, ks, vs, _ = host if host is not None else host_caches(batch)
    dev = batch.q.device
    return (torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev),
            batch.k_scale.to(dev).contiguous(), batch.v_scale.to(dev).contiguous())


def run_step(pa, batch, caches, want_lse=False, stream=None):
    """kv_append of the step's new tokens, then paged_attn_forward."""
    k, v, ks, vs = caches
    c = pa.make_cache(k, v, ks, vs)
    dev = batch.q.device
    pa.kv_append(c, batch.k_new, batch.v_new, batch.slot_mapping.to(dev), stream=stream)
    out, lse = forward(pa, batch, c, want_lse, stream)
    return out, lse, c


def forward(pa, batch, c, want_lse=False, stream=None, q=None, hist=None, incr=None):
    q = batch.q if q is None else q
    hist = batch.hist if hist is None else hist
    incr = batch.incr if incr is None else incr
    dev = q.device
    spec = batch.spec
    bt = torch.from_numpy(batch.block_tables).to(dev)
    ws_bytes = pa.pa_workspace_size(hist, incr, spec.num_q_heads, c)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.full((q.shape[0], spec.num_q_heads, spec.head_dim), float("nan"),
                     dtype=torch.bfloat16, device=dev)
    lse = torch.full((q.shape[0], spec.num_q_heads), float("nan"), dtype=torch.float32,
                     device=dev) if want_lse else None
    pa.paged_attn_forward(q, c, bt, hist, incr, spec.scale, out, ws, lse_out=lse, stream=stream)
    return out, lse
