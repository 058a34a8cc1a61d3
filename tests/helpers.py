"""Test-side helpers: host copies of generated inputs and oracle calls."""
import numpy as np
import torch

import oracle


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bytes8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def host_caches(batch):
    """Host caches holding the batch's history, in the KV storage type.

    bf16: the pool bits.  e4m3: the history encoded by the oracle's codec with
    the batch's scales (NaN slots become the NaN code)."""
    kb, vb = bits16(batch.k_pool), bits16(batch.v_pool)
    if batch.spec.kv_dtype == "bf16":
        return kb.copy(), vb.copy(), None, None, oracle.KV_BF16
    ks = batch.k_scale.detach().cpu().numpy().astype(np.float32)
    vs = batch.v_scale.detach().cpu().numpy().astype(np.float32)
    return oracle.quantize_pool(kb, ks), oracle.quantize_pool(vb, vs), ks, vs, oracle.KV_E4M3


def oracle_step(batch, rows=None, caches=None):
    """Oracle kv_append of the step's new tokens, then oracle attention.

    Returns (out f64, lse f64, caches-after-append)."""
    kc, vc, ks, vs, dt = caches if caches is not None else host_caches(batch)
    oracle.kv_append(kc, vc, ks, vs, dt, bits16(batch.k_new), bits16(batch.v_new),
                     batch.slot_mapping.cpu().numpy())
    out, lse = oracle.attention(bits16(batch.q), kc, vc, ks, vs, dt, batch.block_tables,
                                batch.hist, batch.incr, batch.spec.num_q_heads,
                                batch.spec.scale, rows=rows)
    return out, lse, (kc, vc, ks, vs, dt)


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """float array -> bf16 bit patterns (round-to-nearest-even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
