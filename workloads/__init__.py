"""Seeded synthetic inputs for paged-KV GQA attention.

Shared by the tests, the smoke check and the benchmark.  This module only
*draws* inputs: sequence lengths, the placement of logical blocks in a
physical pool (the KV-cache manager's job, which sits outside the attention
path), slot numbers for the new tokens, and N(0,1) values rounded to bf16.  It
never appends, quantises, gathers or attends: none of the method's arithmetic
lives here.

Shapes and statistics follow the agentic workloads on the pages (page titles
cited in full):
  - "vLLM Agentic 推理｜面向 Agent 负载的推理优化" §2.1: one session's context
    grows 45.7K -> 48.4K -> ... -> 141.5K tokens; sub-agents start from about
    10K tokens of the main agent's context and grow to 29.4K / 59.3K.
  - same page §3.1: median input 142K tokens per request; §3: contexts up to
    1M tokens.
  - "ICML'26 | AMPD ..." §1/§3: incremental prefill of l_incr new tokens over
    l_hist cached ones; initial prefill is l_hist = 0; decode adds one token.
  - "vLLM/V1 推理调度器" 处理流程: one scheduler step shares a token budget
    between running (decode) and newly admitted (prefill) requests.

Random streams: numpy PCG64 seeded by SeedSequence([cfg, stream, ...]) for
lengths (stream 0), block placement (stream 1) and needle placement (6); torch
generators seeded from the same SeedSequence family for q (2), k (3), v (4) and
decode-step tokens (5).

K/V history values are drawn per sequence in logical order and then placed, so
two batches that differ only in placement hold identical logical content.
Every pool slot that holds no history token (spare blocks, tail slots, the
slots the step's new tokens will fill) is poisoned with NaN.

Needles (parity inputs only): a chosen (query row, head) gets one history key
equal to twice its own query vector (exact in bf16), at a seeded history
position.  Its logit, scale * 2 |q|^2 ~ 22.6 at d 128, outweighs the other keys'
N(0, 1) logits even over a million keys, so that row's output is close to the
needle's value vector (|o| ~ 1 instead of ~ sqrt(e / n)): an output computed
from the wrong blocks, or not at all, is then far outside any tolerance.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

BF16_NAN = float("nan")


def _seed(*key) -> int:
    ss = np.random.SeedSequence([int(k) for k in key])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def _np_rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _torch_gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


def randn_bf16(shape, device, *key, chunk_elems: int = 1 << 26, std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) fp32 draws rounded to bf16 (round-to-nearest-even), chunked."""
    g = _torch_gen(device, *key)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        flat[s:e] = x.to(torch.bfloat16)
    return out


@dataclass
class Spec:
    """Lengths and structure of one scheduler step (one layer)."""
    name: str
    cfg: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    hist: List[int]
    incr: List[int]
    kv_dtype: str = "bf16"           # "bf16", "e4m3" or "mxfp4" (the pools hold bf16 values either way)
    shared_prefix_tokens: int = 0    # tokens shared (same physical blocks) by `shared_seqs`
    shared_seqs: List[int] = field(default_factory=list)
    spare_frac: float = 0.01         # extra unreferenced (poisoned) blocks in the pool
    perm_seed: int = 0               # placement stream variant (permutation tests)
    pool_blocks: Optional[int] = None  # force an exact pool size (C1: 18 blocks)
    extra_blocks_per_seq: int = 0    # table capacity beyond the current context
    scale_tokens: Optional[List[int]] = None  # e4m3: scales cover content up to this length
    q_std: float = 1.0               # standard deviation of q (logit std ~ q_std)
    needles: List[Tuple[int, int]] = field(default_factory=list)  # (seq, row of its increment)
    decode_needle_steps: List[int] = field(default_factory=list)  # single-session decode steps

    @property
    def num_seqs(self):
        return len(self.hist)

    @property
    def total_q(self):
        return int(sum(self.incr))

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


@dataclass
class Batch:
    spec: Spec
    block_tables: np.ndarray      # int32 [num_seqs, max_blocks], padded with -1
    num_blocks: int               # physical pool size
    hist: np.ndarray              # int32 [num_seqs]
    incr: np.ndarray              # int32 [num_seqs]
    slot_mapping: torch.Tensor    # int64 [total_q]
    q: torch.Tensor               # bf16 [total_q, Hq, d]
    k_new: torch.Tensor           # bf16 [total_q, Hkv, d]
    v_new: torch.Tensor           # bf16 [total_q, Hkv, d]
    k_pool: torch.Tensor          # bf16 [nb, Hkv, bs, d]: history values, NaN elsewhere
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor] = None   # fp32 [nb, Hkv] (e4m3 only)
    v_scale: Optional[torch.Tensor] = None
    # planted needles: (global q row, q head, seq, history position); decode-step
    # needles: {step: (q head, history position)}
    needles: List[Tuple[int, int, int, int]] = field(default_factory=list)
    decode_needles: dict = field(default_factory=dict)

    @property
    def max_blocks(self):
        return self.block_tables.shape[1]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _place(spec: Spec, ctx_alloc: List[int]):
    """Assign physical block ids: the KV-cache manager's role (out of the path)."""
    bs = spec.block_size
    nblk = [_ceil_div(c, bs) for c in ctx_alloc]
    shared = _ceil_div(spec.shared_prefix_tokens, bs) if spec.shared_seqs else 0
    if shared:
        assert spec.shared_prefix_tokens % bs == 0, "shared prefix must be whole blocks"
    own = [n - (shared if s in spec.shared_seqs else 0) for s, n in enumerate(nblk)]
    need = shared + sum(own)
    pool = spec.pool_blocks or need + max(1, int(math.ceil(need * spec.spare_frac)))
    assert pool >= need
    perm = _np_rng(spec.cfg, 1, spec.perm_seed).permutation(pool).astype(np.int32)
    cur = 0
    shared_ids = perm[cur:cur + shared]
    cur += shared
    max_blocks = max(nblk) + spec.extra_blocks_per_seq if nblk else 1
    bt = np.full((spec.num_seqs, max(max_blocks, 1)), -1, dtype=np.int32)
    for s in range(spec.num_seqs):
        row = []
        if s in spec.shared_seqs:
            row.extend(shared_ids.tolist())
        row.extend(perm[cur:cur + own[s]].tolist())
        cur += own[s]
        bt[s, :len(row)] = row
    return bt, pool, shared


def make_batch(spec: Spec, device="cpu") -> Batch:
    """Draw one step's inputs.  Pools hold history tokens [0, hist) only."""
    bs, hkv, d, hq = spec.block_size, spec.num_kv_heads, spec.head_dim, spec.num_q_heads
    hist = np.asarray(spec.hist, dtype=np.int32)
    incr = np.asarray(spec.incr, dtype=np.int32)
    ctx = [int(h) + int(n) for h, n in zip(hist, incr)]
    scale_ctx = spec.scale_tokens if spec.scale_tokens is not None else ctx
    alloc_ctx = [max(a, b) for a, b in zip(ctx, scale_ctx)]
    bt, pool, shared_blocks = _place(spec, alloc_ctx)
    total_q = spec.total_q

    k_pool = torch.full((pool, hkv, bs, d), BF16_NAN, dtype=torch.bfloat16, device=device)
    v_pool = torch.full((pool, hkv, bs, d), BF16_NAN, dtype=torch.bfloat16, device=device)

    def fill_history(pool_t, stream):
        done_shared = False
        for s in range(spec.num_seqs):
            h = int(hist[s])
            nb_s = _ceil_div(h, bs)
            start_blk = 0
            if s in spec.shared_seqs and shared_blocks:
                if not done_shared:
                    vals = randn_bf16((shared_blocks, hkv, bs, d), device, spec.cfg, stream, 0)
                    ids = torch.as_tensor(bt[s, :shared_blocks], dtype=torch.long, device=device)
                    pool_t[ids] = vals
                    done_shared = True
                start_blk = shared_blocks
                assert h >= spec.shared_prefix_tokens
            nb_own = nb_s - start_blk
            if nb_own <= 0:
                continue
            vals = randn_bf16((nb_own, hkv, bs, d), device, spec.cfg, stream, 1, s)
            tail = h - (nb_s - 1) * bs  # valid tokens in the last history block
            if tail < bs:
                vals[-1, :, tail:, :] = BF16_NAN
            ids = torch.as_tensor(bt[s, start_blk:nb_s], dtype=torch.long, device=device)
            pool_t[ids] = vals

    fill_history(k_pool, 3)
    fill_history(v_pool, 4)

    q = randn_bf16((total_q, hq, d), device, spec.cfg, 2, std=spec.q_std)
    k_new = randn_bf16((total_q, hkv, d), device, spec.cfg, 3, 2)
    v_new = randn_bf16((total_q, hkv, d), device, spec.cfg, 4, 2)

    slots = np.empty(total_q, dtype=np.int64)
    r = 0
    for s in range(spec.num_seqs):
        for p in range(int(hist[s]), int(hist[s]) + int(incr[s])):
            slots[r] = int(bt[s, p // bs]) * bs + p % bs
            r += 1
    slot_mapping = torch.as_tensor(slots, device=device)

    b = Batch(spec, bt, pool, hist, incr, slot_mapping, q, k_new, v_new, k_pool, v_pool)
    if spec.needles or spec.decode_needle_steps:
        _plant_needles(b)
    if spec.kv_dtype == "e4m3":
        b.k_scale, b.v_scale = _amax_scales(b, scale_ctx)
    return b


def _plant_needles(b: Batch):
    """Set one seeded history key per needle to 2 x the needled query vector
    (a power-of-two multiple: exact in bf16).  Positions are distinct."""
    spec = b.spec
    bs, G = spec.block_size, spec.num_q_heads // spec.num_kv_heads
    rng = _np_rng(spec.cfg, 6, spec.perm_seed)
    rowstart = np.concatenate([[0], np.cumsum(b.incr.astype(np.int64))])
    used = set()

    def plant(seq, qvec_heads, what):
        h = int(rng.integers(0, spec.num_q_heads))
        hist = int(b.hist[seq])
        assert hist > 0, f"needle {what} needs a history"
        while True:
            j = int(rng.integers(0, hist))
            if (seq, j) not in used:
                break
        used.add((seq, j))
        phys = int(b.block_tables[seq, j // bs])
        key = (2 * qvec_heads[h].float()).to(torch.bfloat16)
        b.k_pool[phys, h // G, j % bs, :] = key
        return h, j

    for seq, i in spec.needles:
        assert 0 <= i < int(b.incr[seq])
        row = int(rowstart[seq]) + i
        h, j = plant(seq, b.q[row], f"({seq}, {i})")
        b.needles.append((row, h, seq, j))
    for step in spec.decode_needle_steps:
        q, _, _ = decode_step_tokens(spec, step, b.q.device)
        b.decode_needles[step] = plant(0, q[0], f"step {step}")


def with_needles(spec: Spec, needles=(), decode_steps=(), q_std: float = None) -> Spec:
    """A copy of `spec` with planted needles (parity inputs)."""
    import dataclasses
    kw = dict(needles=list(needles), decode_needle_steps=list(decode_steps))
    if q_std is not None:
        kw["q_std"] = q_std
    return dataclasses.replace(spec, **kw)


def decode_step_tokens(spec: Spec, step: int, device="cpu"):
    """Fresh N(0,1) q/k/v for one decode step of a single session (stream 5)."""
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    q = randn_bf16((1, hq, d), device, spec.cfg, 5, step, 0)
    k = randn_bf16((1, hkv, d), device, spec.cfg, 5, step, 1)
    v = randn_bf16((1, hkv, d), device, spec.cfg, 5, step, 2)
    return q, k, v


def _amax_scales(b: Batch, scale_ctx):
    """Per-(block, KV head) E4M3 scales: amax/448 over the block's final content
    (history plus every token later appended into it), 1.0 where amax is 0.
    The caller's quantisation policy, drawn with the inputs."""
    spec = b.spec
    bs = spec.block_size
    dev = b.k_pool.device
    ks = torch.zeros((b.num_blocks, spec.num_kv_heads), dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)

    def blk_amax(pool):
        return torch.nan_to_num(pool.float(), nan=0.0).abs().amax(dim=(2, 3))

    ks = torch.maximum(ks, blk_amax(b.k_pool))
    vs = torch.maximum(vs, blk_amax(b.v_pool))
    # the step's new tokens
    slots = b.slot_mapping.long()
    blk = slots // bs
    ks.index_reduce_(0, blk, b.k_new.float().abs().amax(dim=2), "amax")
    vs.index_reduce_(0, blk, b.v_new.float().abs().amax(dim=2), "amax")
    # later decode tokens (single-session long-context decode)
    if spec.num_seqs == 1 and scale_ctx[0] > int(b.hist[0]) + int(b.incr[0]):
        first = int(b.hist[0]) + int(b.incr[0])
        for step, p in enumerate(range(first, scale_ctx[0])):
            _, k, v = decode_step_tokens(spec, step + 1, dev)
            pb = int(b.block_tables[0, p // bs])
            ks[pb] = torch.maximum(ks[pb], k[0].float().abs().amax(dim=1))
            vs[pb] = torch.maximum(vs[pb], v[0].float().abs().amax(dim=1))
    ks = torch.where(ks > 0, ks / 448.0, torch.ones_like(ks))
    vs = torch.where(vs > 0, vs / 448.0, torch.ones_like(vs))
    return ks.contiguous(), vs.contiguous()


# ---------------------------------------------------------------------------
# The five workloads (one layer each) and their variants.

def lognormal_ctx(rng: np.random.Generator, n: int, median: float, sigma: float, lo: int, hi: int):
    z = rng.standard_normal(n)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)


def tiny(perm_seed: int = 0) -> Spec:
    """1 session, 4 q / 1 KV head, d 64, bs 16, hist 256 + incr 32; the table is a
    seeded permutation of exactly 18 physical blocks."""
    return Spec("tiny", 1, 4, 1, 64, 16, [256], [32], pool_blocks=18, perm_seed=perm_seed)


def incremental(hist: int = 45_700, incr: int = 2_700, name: str = "incremental_prefill",
                block_size: int = 16) -> Spec:
    """Single-session incremental prefill, 32 q / 8 KV heads, d 128 (45.7K -> 48.4K)."""
    return Spec(name, 2, 32, 8, 128, block_size, [hist], [incr])


def initial(tokens: int = 45_700) -> Spec:
    return Spec("initial_prefill", 2, 32, 8, 128, 16, [0], [tokens])


def decode_batch(num_sessions: int = 64, median: float = 142_000.0, sigma: float = 0.5,
                 lo: int = 10_000, hi: int = 262_144, cfg: int = 3) -> Spec:
    """Batched decode: lognormal contexts (median 142K, sigma 0.5, clipped)."""
    ctx = lognormal_ctx(_np_rng(cfg, 0), num_sessions, median, sigma, lo, hi)
    hist = [int(c) - 1 for c in ctx]
    return Spec("decode_batch", cfg, 32, 8, 128, 16, hist, [1] * num_sessions)


def mixed(cfg: int = 4, budget: int = 8192) -> Spec:
    """Mixed step: 4 incremental prefills + 48 decodes (8 sub-agents sharing a
    10,000-token prefix, 40 with lognormal contexts), one token budget."""
    rng = _np_rng(cfg, 0)
    while True:
        pre_incr = rng.integers(256, 4096, size=4, endpoint=True)
        if int(pre_incr.sum()) + 48 <= budget:
            break
    pre_hist = lognormal_ctx(rng, 4, 100_000.0, 0.5, 10_000, 262_144)
    sub_ctx = 10_000 + rng.integers(20_000, 50_000, size=8, endpoint=True)
    dec_ctx = lognormal_ctx(rng, 40, 142_000.0, 0.5, 10_000, 262_144)
    hist = [int(h) for h in pre_hist] + [int(c) - 1 for c in sub_ctx] + [int(c) - 1 for c in dec_ctx]
    incr = [int(n) for n in pre_incr] + [1] * 48
    return Spec("mixed", cfg, 32, 8, 128, 16, hist, incr, shared_prefix_tokens=10_000,
                shared_seqs=list(range(4, 12)))


def long_context(hist: int = 1_044_480, incr: int = 4_096, decode_steps: int = 256) -> Spec:
    """1 session, 1M-token history, fp8 E4M3 KV with per-(block, head) scales, bs 64."""
    total = hist + incr + decode_steps
    return Spec("long_context", 5, 32, 8, 128, 64, [hist], [incr], kv_dtype="e4m3",
                scale_tokens=[total], extra_blocks_per_seq=0)



def long_context_mxfp4(hist: int = 1_044_480, incr: int = 4_096, decode_steps: int = 256) -> Spec:
    """The 1M-token session with 4-bit KV: OCP MXFP4 (E2M1 codes, one E8M0
    scale per 32 elements of a token and head), bs 64.  The scales are derived
    from the values when they are encoded, so the spec carries none."""
    return Spec("long_context_mxfp4", 5, 32, 8, 128, 64, [hist], [incr], kv_dtype="mxfp4",
                scale_tokens=[hist + incr + decode_steps], extra_blocks_per_seq=0)


def slot_of(batch: Batch, seq: int, pos: int) -> int:
    """Cache slot (physical block * block_size + offset) of a token position,
    as the KV-cache manager hands it to the attention layer."""
    bs = batch.spec.block_size
    return int(batch.block_tables[seq, pos // bs]) * bs + pos % bs
