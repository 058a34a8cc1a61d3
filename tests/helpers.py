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
    the batch's scales (NaN slots become the NaN code).  mxfp4: the history
    encoded by the oracle's MXFP4 encoder (unwritten slots, NaN in the pool,
    get the NaN scale and zero codes)."""
    kb, vb = bits16(batch.k_pool), bits16(batch.v_pool)
    if batch.spec.kv_dtype == "bf16":
        return kb.copy(), vb.copy(), None, None, oracle.KV_BF16
    if batch.spec.kv_dtype == "mxfp4":
        kc, ks = oracle.mxfp4_quantize_pool(kb)
        vc, vs = oracle.mxfp4_quantize_pool(vb)
        return kc, vc, ks, vs, oracle.KV_MXFP4
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


_E4M3_LUT = None


def key_values(caches, bt_row, ctx):
    """Values [ctx, hkv, d] (fp64) of one sequence's keys from host caches,
    through the oracle's gather and its codecs (test-side bound computations)."""
    global _E4M3_LUT
    kc, _, ks, _, dt = caches
    if dt == oracle.KV_MXFP4:
        return oracle.gather_values(kc, ks, dt, bt_row, ctx)
    raw = oracle.gather(kc, bt_row, ctx)
    if dt == oracle.KV_BF16:
        return bf16_values(raw)
    if _E4M3_LUT is None:
        _E4M3_LUT = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    bs = kc.shape[2]
    blk = bt_row[np.arange(ctx) // bs]
    return _E4M3_LUT[raw] * ks[blk][:, :, None].astype(np.float64)


def row_paths(batch):
    """Per q row, the kernel family that computes it: 'w48' (the 384-row
    prefill, head dim 128: l summed from bf16-rounded probabilities) or
    'exact' (decode kernels and the head-dim-64 prefill: fp32 probability sums)."""
    spec = batch.spec
    G = spec.num_q_heads // spec.num_kv_heads
    out = []
    for s in range(spec.num_seqs):
        n = int(batch.incr[s])
        decode_class = n <= 16 // G
        out += ["w48" if (spec.head_dim == 128 and not decode_class) else "exact"] * n
    return out


def lse_bounds(batch, caches):
    """Per (q row, head) LSE bound [total_q, hq] for the row's kernel family."""
    from tests.parity import LSE_EXACT, w48_lse_bound
    spec = batch.spec
    G = spec.num_q_heads // spec.num_kv_heads
    fp8 = spec.kv_dtype == "e4m3"
    paths = row_paths(batch)
    bound = np.full((spec.total_q, spec.num_q_heads), LSE_EXACT)
    q = bf16_values(bits16(batch.q))
    r0 = 0
    for s in range(spec.num_seqs):
        n = int(batch.incr[s])
        if n and paths[r0] == "w48":
            if not fp8:
                bound[r0:r0 + n] = w48_lse_bound(q[r0:r0 + 1, 0], None, spec.scale, False)[0]
            else:
                ctx = int(batch.hist[s]) + n
                keys = key_values(caches, batch.block_tables[s], ctx)
                for h in range(spec.num_q_heads):
                    bound[r0:r0 + n, h] = w48_lse_bound(q[r0:r0 + n, h], keys[:, h // G], spec.scale, True)
        r0 += n
    return bound
