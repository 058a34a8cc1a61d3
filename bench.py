#!/usr/bin/env python3
"""Benchmark of the paged-KV GQA attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input: kv_append of the
step's new tokens into their cache slots, then paged_attn_forward (work
planner, attention kernel(s), LSE merge).  Inputs are resident in HBM before
the timed region.

Default workload (the headline): single-session incremental prefill, one
layer, 32 q / 8 KV heads, head_dim 128, block 16, bf16: 45,700 cached tokens,
2,700 new (a 45.7K -> 48.4K agent turn).  `value` is its attention TFLOP/s
(4 * d * Hq flops per unmasked (query, key) pair) over the whole step.  Also
measured in the same run and reported as sub-objects: batched decode (64
sessions, lognormal contexts with median 142K) in KV GB/s, and incremental
prefill at 128K history.  Unless --no-reports, `reports` carries the other
workloads of the same path, each timed the same way: initial prefill of
45,700 tokens, the 128K history with 4,096 new tokens, a mixed step (4
incremental prefills + 48 decodes, 8 of them over a shared 10,000-token
prefix), the 1M-token E4M3 history (incremental prefill of 4,096 tokens and a
decode step at 1,048,576), and kv_append bandwidth.  The oracle's CPU rate on
a bounded sample of the headline workload is reported as `cpu_baseline`.

Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "incremental-prefill attn TFLOP/s + decode KV GB/s, % of MI355X roofline"


def prefill_flops(hist, incr, hq, d):
    """4 * d * Hq flops per unmasked (query, key) pair."""
    pairs = sum(int(n) * int(h) + int(n) * (int(n) + 1) // 2 for h, n in zip(hist, incr))
    return 4 * d * hq * pairs


def kv_bytes_per_token(spec):
    """K and V bytes of one token, all KV heads: bf16 2 per element, E4M3 1
    (its per-(block, head) scales are under 0.1%), MXFP4 half a byte plus
    one scale byte per 32 elements."""
    if spec.kv_dtype == "mxfp4":
        return 2 * spec.num_kv_heads * (spec.head_dim // 2 + spec.head_dim // 32)
    elem = 1 if spec.kv_dtype == "e4m3" else 2
    return 2 * spec.num_kv_heads * spec.head_dim * elem


def decode_bytes(spec):
    """Algorithmic HBM bytes the decode attention moves in one step: every
    context token's K and V read once (the step's own token included), plus q
    read, out written and the block-table entries read.  (The append of the
    step's token is kv_append's traffic, reported on its own.)"""
    ctx = sum(int(h) + int(n) for h, n in zip(spec.hist, spec.incr))
    q = spec.total_q * spec.num_q_heads * spec.head_dim * 2
    nb = sum(-(-(int(h) + int(n)) // spec.block_size) for h, n in zip(spec.hist, spec.incr))
    return ctx * kv_bytes_per_token(spec) + 2 * q + nb * 4


def prefill_bytes(spec):
    ctx = sum(int(h) + int(n) for h, n in zip(spec.hist, spec.incr))
    q = spec.total_q * spec.num_q_heads * spec.head_dim * 2
    return ctx * kv_bytes_per_token(spec) + 2 * q


class Runner:
    """Holds one workload's device inputs and runs steps through the C ABI."""

    def __init__(self, pa, torch, spec, dev):
        import workloads as W
        self.pa, self.torch, self.spec = pa, torch, spec
        b = W.make_batch(spec, dev)
        self.b = b
        if spec.kv_dtype == "e4m3":
            # E4M3 codes of the history under the per-(block, head) scales
            # (input preparation; the step's own tokens go through kv_append)
            def codes(pool, sc):
                out = torch.empty(pool.shape, dtype=torch.uint8, device=dev)
                for i in range(0, pool.shape[0], 4096):
                    x = pool[i:i + 4096].float() / sc[i:i + 4096, :, None, None]
                    out[i:i + 4096] = x.to(torch.float8_e4m3fn).view(torch.uint8)
                return out
            self.k_codes, self.v_codes = codes(b.k_pool, b.k_scale), codes(b.v_pool, b.v_scale)
            b.k_pool = b.v_pool = None
            torch.cuda.empty_cache()
            self.cache = pa.make_cache(self.k_codes, self.v_codes, b.k_scale, b.v_scale)
        elif spec.kv_dtype == "mxfp4":
            # the history encoded by the library's own quantising kv_append,
            # a block range at a time (unwritten slots, NaN in the pool, get
            # the NaN scale and zero codes)
            nb, hkv, bs, d = b.k_pool.shape
            self.k_codes = torch.empty((nb, hkv, bs, d // 2), dtype=torch.uint8, device=dev)
            self.v_codes = torch.empty_like(self.k_codes)
            self.k_sc = torch.empty((nb, hkv, d // 32, bs), dtype=torch.uint8, device=dev)
            self.v_sc = torch.empty_like(self.k_sc)
            self.cache = pa.make_cache(self.k_codes, self.v_codes, self.k_sc, self.v_sc)
            for i in range(0, nb, 4096):
                j = min(nb, i + 4096)
                kt = b.k_pool[i:j].permute(0, 2, 1, 3).reshape((j - i) * bs, hkv, d).contiguous()
                vt = b.v_pool[i:j].permute(0, 2, 1, 3).reshape((j - i) * bs, hkv, d).contiguous()
                pa.kv_append(self.cache, kt, vt, torch.arange(i * bs, j * bs, dtype=torch.int64, device=dev))
            torch.cuda.synchronize()
            b.k_pool = b.v_pool = None
            torch.cuda.empty_cache()
        else:
            self.cache = pa.make_cache(b.k_pool, b.v_pool)
        self.bt = torch.from_numpy(b.block_tables).to(dev)
        self.slots = b.slot_mapping.to(dev)
        ws = pa.pa_workspace_size(b.hist, b.incr, spec.num_q_heads, self.cache)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.out = torch.empty((spec.total_q, spec.num_q_heads, spec.head_dim),
                               dtype=torch.bfloat16, device=dev)
        self.stream = torch.cuda.current_stream()

    def use_cascade(self):
        """Run steps through paged_attn_forward_cascade with the workload's
        shared-prefix group declared (the sub-agents of the mixed step)."""
        spec, b, pa = self.spec, self.b, self.pa
        self.group_of = [0 if s in spec.shared_seqs else -1 for s in range(spec.num_seqs)]
        self.group_len = [spec.shared_prefix_tokens]
        need = pa.cascade_workspace_size(b.hist, b.incr, spec.num_q_heads, self.cache, self.bt,
                                         self.group_of, self.group_len, spec.scale)
        self.ws = self.torch.empty(need, dtype=self.torch.uint8, device=self.ws.device)
        self.cascade = True

    def use_one_launch(self):
        """Run steps through paged_attn_step (kv_append and the attention in
        one persistent launch)."""
        spec, b, pa = self.spec, self.b, self.pa
        need = pa.step_workspace_size(b.hist, b.incr, spec.num_q_heads, self.cache, self.bt, spec.scale)
        self.ws = self.torch.empty(need, dtype=self.torch.uint8, device=self.ws.device)
        self.one_launch = True

    def step(self):
        b, pa = self.b, self.pa
        if getattr(self, "one_launch", False):
            pa.paged_attn_step(self.cache, b.k_new, b.v_new, self.slots, b.q, self.bt, b.hist, b.incr,
                               self.spec.scale, self.out, self.ws, stream=self.stream)
            return
        pa.kv_append(self.cache, b.k_new, b.v_new, self.slots, stream=self.stream)
        if getattr(self, "cascade", False):
            pa.paged_attn_forward_cascade(b.q, self.cache, self.bt, b.hist, b.incr, self.spec.scale,
                                          self.out, self.ws, self.group_of, self.group_len,
                                          stream=self.stream)
            return
        pa.paged_attn_forward(b.q, self.cache, self.bt, b.hist, b.incr, self.spec.scale, self.out,
                              self.ws, stream=self.stream)

    def timed(self, steps, warmup):
        """(ms per step, {kernel: (ms per launch, launches per step)}).  After
        the warm-up, a pass of the steps with HIP events around each launch
        gives the kernel times; the step time comes from the timed pass that
        follows, without per-launch events (they cost ~10 us per step)."""
        torch, pa = self.torch, self.pa
        # warm-up: W steps, and at least ~150 ms of them (the clock settles)
        t0 = time.time()
        n = 0
        while n < warmup or time.time() - t0 < 0.15:
            self.step()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        for k in range(pa.TIMING_KINDS):
            pa.pa_timing_read(k)  # drop anything recorded before
        pa.pa_timing_enable(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        pa.pa_timing_enable(False)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(steps):
            self.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        kern = {}
        for kind, name in ((0, "kv_append"), (1, "prefill"), (2, "decode"), (3, "merge"), (4, "step")):
            tot, cnt = pa.pa_timing_read(kind)
            if cnt:
                kern[name] = (tot / cnt, cnt / steps)   # avg ms per launch, launches per step
        return ms, kern


def _kern(kern):
    return {k: round(v[0], 4) for k, v in kern.items()}


def report_prefill(pa, torch, spec, dev, steps, warmup, label, runner=None):
    r = runner or Runner(pa, torch, spec, dev)
    ms, kern = r.timed(steps, warmup)
    fl = prefill_flops(spec.hist, spec.incr, spec.num_q_heads, spec.head_dim)
    k_ms = kern["prefill"][0] * kern["prefill"][1]
    d = {"workload": label, "ms_per_step": round(ms, 4),
         "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
         "tokens_per_s": round(spec.total_q / (ms * 1e-3), 1),
         "kernels_ms": _kern(kern),
         "roofline": {"bound": "mfma", "achieved": round(fl / (k_ms * 1e-3) / 1e12, 2),
                      "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(fl / (k_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "kernel": "prefill_w48_kernel<%d, %d>" % (
                          spec.block_size, {"bf16": 0, "e4m3": 1, "mxfp4": 2}[spec.kv_dtype])}}
    if runner is None:
        del r
        torch.cuda.empty_cache()
    return d


def report_decode_steps(pa, torch, r, dev, label, nsteps=256, warmup=16):
    """The decode steps that follow an incremental prefill of one session: step
    j appends one token at position hist + incr + j - 1 and attends over the
    whole context.  The steps are run as a serving loop would (each plans on
    the host and launches); one pass with HIP events around each launch gives
    the kernel times, then a clean pass with one event per step gives each
    step's time (median, min, max) and the total.  Re-running a step rewrites
    the same bytes, so passes are repeatable."""
    import workloads as W
    spec, b = r.spec, r.b
    first = int(b.hist[0]) + int(b.incr[0])
    r.step()  # the prefill's own tokens are in the cache
    toks = [W.decode_step_tokens(spec, j, dev) for j in range(1, nsteps + 1)]
    slots = [torch.tensor([W.slot_of(b, 0, first + j - 1)], dtype=torch.int64, device=dev)
             for j in range(1, nsteps + 1)]
    hists = [np.array([first + j - 1], np.int32) for j in range(1, nsteps + 1)]
    one = np.array([1], np.int32)
    ws_need = pa.pa_workspace_size(hists[-1], one, spec.num_q_heads, r.cache)
    ws = r.ws if r.ws.numel() >= ws_need else torch.empty(ws_need, dtype=torch.uint8, device=dev)
    out = torch.empty((1, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device=dev)

    def step(j):
        q, k, v = toks[j]
        pa.kv_append(r.cache, k, v, slots[j], stream=r.stream)
        pa.paged_attn_forward(q, r.cache, r.bt, hists[j], one, spec.scale, out, ws, stream=r.stream)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    for k in range(pa.TIMING_KINDS):
        pa.pa_timing_read(k)
    pa.pa_timing_enable(True)
    for j in range(nsteps):
        step(j)
    torch.cuda.synchronize()
    pa.pa_timing_enable(False)
    kern = {}
    for kind, name in ((0, "kv_append"), (2, "decode"), (3, "merge")):
        tot, cnt = pa.pa_timing_read(kind)
        if cnt:
            kern[name] = (tot / cnt, cnt / nsteps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    ev[0].record(r.stream)
    for j in range(nsteps):
        step(j)
        ev[j + 1].record(r.stream)
    torch.cuda.synchronize()
    per = np.array([ev[j].elapsed_time(ev[j + 1]) for j in range(nsteps)])
    total = ev[0].elapsed_time(ev[nsteps])
    med = float(np.median(per))
    # algorithmic bytes of the middle step (the steps differ by < 0.03%)
    mid = W.Spec(spec.name, spec.cfg, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                 spec.block_size, [first + nsteps // 2 - 1], [1], kv_dtype=spec.kv_dtype)
    byts = decode_bytes(mid)
    k_ms = kern["decode"][0] * kern["decode"][1] + kern.get("merge", (0, 0))[0] * kern.get("merge", (0, 0))[1]
    dk_ms = kern["decode"][0] * kern["decode"][1]
    return {"workload": label, "steps": nsteps,
            "ms_per_step_median": round(med, 4), "ms_per_step_min": round(float(per.min()), 4),
            "ms_per_step_max": round(float(per.max()), 4), "total_ms": round(total, 3),
            "GB/s_median_step": round(byts / (med * 1e-3) / 1e9, 1),
            "tokens_per_s": round(nsteps / (total * 1e-3), 1),
            "kernels_ms": _kern(kern), "decode_plus_merge_ms": round(k_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(byts / (dk_ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(byts / (dk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(f"decode_long_{spec.kv_dtype}_bytes"),
                         "algorithmic_bytes": int(byts),
                         "kernel": {"e4m3": "decode_dma_fp8_kernel<64, 8, 2>",
                                    "mxfp4": "decode_dma_fp4_kernel<64, 8, 2>"}.get(spec.kv_dtype)}}


def report_decode(pa, torch, spec, dev, steps, warmup, label, kernel=None, traffic_key=None):
    r = Runner(pa, torch, spec, dev)
    ms, kern = r.timed(steps, warmup)
    byts = decode_bytes(spec)
    k_ms = kern["decode"][0] * kern["decode"][1]
    d = {"workload": label, "ms_per_step": round(ms, 4),
         "GB/s": round(byts / (ms * 1e-3) / 1e9, 1),
         "tokens_per_s": round(spec.total_q / (ms * 1e-3), 1),
         "kernels_ms": _kern(kern),
         "roofline": {"bound": "hbm", "achieved": round(byts / (k_ms * 1e-3) / 1e9, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(byts / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic(traffic_key) if traffic_key else None,
                      "algorithmic_bytes": int(byts), "kernel": kernel}}
    del r
    torch.cuda.empty_cache()
    return d


def mixed_parts(spec):
    """(prefill flops, decode flops, decode unique bytes) of a mixed step: the
    sequences with more than one new token are prefills, the rest decodes;
    the shared prefix's blocks are counted once."""
    pre = [i for i, n in enumerate(spec.incr) if n > 1]
    dec = [i for i, n in enumerate(spec.incr) if n == 1]
    fl = prefill_flops([spec.hist[i] for i in pre], [spec.incr[i] for i in pre],
                       spec.num_q_heads, spec.head_dim)
    dfl = prefill_flops([spec.hist[i] for i in dec], [1] * len(dec), spec.num_q_heads, spec.head_dim)
    kvb = kv_bytes_per_token(spec)
    shared = [i for i in dec if i in spec.shared_seqs]
    uniq = sum(spec.hist[i] + 1 for i in dec) - max(0, len(shared) - 1) * spec.shared_prefix_tokens
    byts = uniq * kvb + 2 * len(dec) * spec.num_q_heads * spec.head_dim * 2
    return fl, dfl, byts


def report_mixed_one_launch(pa, torch, spec, dev, steps, warmup, label):
    """The mixed step through paged_attn_step: one persistent launch (after
    the work-list copy) for the append, both attention parts and the merges."""
    r = Runner(pa, torch, spec, dev)
    r.use_one_launch()
    ms, kern = r.timed(steps, warmup)
    fl, dfl, byts = mixed_parts(spec)
    k_ms = kern["step"][0] * kern["step"][1]
    return {"workload": label, "ms_per_step": round(ms, 4), "kernels_ms": _kern(kern),
            "step_kernel_ms": round(k_ms, 4),
            "note": "prefill and decode parts share the launch: no per-part rates"}


def report_mixed(pa, torch, spec, dev, steps, warmup, label, cascade=False, overlap=None):
    """One call holding 4 incremental prefills and 48 decodes.  Launched one
    after the other (overlap=0, or the cascade entry point): the prefill part
    in TFLOP/s over its kernel, the decode part in GB/s over its kernel (the
    decode launch holds the shared-prefix cascade items when the sub-agents
    are declared as a group; the shared prefix's blocks are counted once
    either way).  Co-scheduled (the planner's choice): the decode's first
    launch runs beside the prefill on a few CUs, so per-kernel rates overlap;
    the parts' rates are given over the whole step instead."""
    if overlap is not None:
        pa.pa_debug_overlap_cus(overlap)
    try:
        r = Runner(pa, torch, spec, dev)
        if cascade:
            r.use_cascade()
        ms, kern = r.timed(steps, warmup)
        groups = pa.pa_debug_plan_groups(spec.hist, spec.incr, spec.num_q_heads, r.cache)
    finally:
        if overlap is not None:
            pa.pa_debug_overlap_cus(-1)
    fl, _, byts = mixed_parts(spec)
    p_ms = kern["prefill"][0] * kern["prefill"][1]
    d = {"workload": label, "ms_per_step": round(ms, 4), "kernels_ms": _kern(kern)}
    if kern["decode"][1] > 1.5:  # co-scheduled: one decode launch beside the prefill, one after
        cus = pa.pa_device_shape()[0]
        n_pre = len(groups) - 1
        d.update({"co_scheduled": {"prefill_cus": n_pre, "decode_cus_beside_prefill": cus - n_pre},
                  "prefill_TFLOP/s_kernel": round(fl / (p_ms * 1e-3) / 1e12, 2),
                  "prefill_TFLOP/s_over_step": round(fl / (ms * 1e-3) / 1e12, 2),
                  "decode_GB/s_over_step": round(byts / (ms * 1e-3) / 1e9, 1),
                  "decode_unique_bytes": int(byts)})
    else:
        d_ms = kern["decode"][0] * kern["decode"][1]
        d.update({"prefill_TFLOP/s_kernel": round(fl / (p_ms * 1e-3) / 1e12, 2),
                  "prefill_frac": round(fl / (p_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "decode_GB/s_kernel": round(byts / (d_ms * 1e-3) / 1e9, 1),
                  "decode_frac": round(byts / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "decode_unique_bytes": int(byts)})
    del r
    torch.cuda.empty_cache()
    return d


def report_append(pa, torch, dev, tokens, steps, label):
    """kv_append of `tokens` bf16 tokens (8 KV heads, d 128, block 16) into
    a pool of exactly those slots, in a seeded permuted block order."""
    import workloads as W
    hkv, d, bs = 8, 128, 16
    nb = (tokens + bs - 1) // bs
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    cache = pa.make_cache(kc, vc)
    k_new = W.randn_bf16((tokens, hkv, d), dev, 90, 3)
    v_new = W.randn_bf16((tokens, hkv, d), dev, 90, 4)
    perm = torch.from_numpy(np.random.default_rng(90).permutation(nb).astype(np.int64)).to(dev)
    pos = torch.arange(tokens, device=dev, dtype=torch.int64)
    slots = perm[pos // bs] * bs + pos % bs
    s = torch.cuda.current_stream()
    pa.kv_append(cache, k_new, v_new, slots, stream=s)
    torch.cuda.synchronize()
    pa.pa_timing_read(0)
    pa.pa_timing_enable(True)
    for _ in range(steps):
        pa.kv_append(cache, k_new, v_new, slots, stream=s)
    torch.cuda.synchronize()
    pa.pa_timing_enable(False)
    tot, cnt = pa.pa_timing_read(0)
    k_ms = tot / cnt
    byts = 2 * tokens * hkv * d * 2 * 2 + tokens * 8   # K and V read and written, slots read
    # a plain device copy of the same K and V bytes, for comparison
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kflat, vflat = kc.view(-1)[:k_new.numel()], vc.view(-1)[:v_new.numel()]
    kflat.copy_(k_new.view(-1))
    e0.record(s)
    for _ in range(steps):
        kflat.copy_(k_new.view(-1))
        vflat.copy_(v_new.view(-1))
    e1.record(s)
    torch.cuda.synchronize()
    c_ms = e0.elapsed_time(e1) / steps
    out = {"workload": label, "tokens": tokens, "kernel_ms": round(k_ms, 4),
           "GB/s": round(byts / (k_ms * 1e-3) / 1e9, 1),
           "frac": round(byts / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": int(byts),
           "plain_copy_GB/s": round(4 * tokens * hkv * d * 2 / (c_ms * 1e-3) / 1e9, 1),
           "traffic": measured_traffic("kv_append_1m_bytes") if tokens == 1_048_576 else None}
    del kc, vc, k_new, v_new
    torch.cuda.empty_cache()
    return out


def report_append_e4m3(pa, torch, dev, tokens, steps, label):
    """The long-context step's quantising kv_append: `tokens` bf16 tokens (8 KV
    heads, d 128) into an E4M3 cache of block 64 with per-(block, head)
    scales, in a seeded permuted block order."""
    import workloads as W
    hkv, d, bs = 8, 128, 64
    nb = (tokens + bs - 1) // bs
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    k_new = W.randn_bf16((tokens, hkv, d), dev, 91, 3)
    v_new = W.randn_bf16((tokens, hkv, d), dev, 91, 4)
    ks = torch.full((nb, hkv), 4.5 / 448, dtype=torch.float32, device=dev)
    vs = torch.full((nb, hkv), 4.5 / 448, dtype=torch.float32, device=dev)
    cache = pa.make_cache(kc, vc, ks, vs)
    perm = torch.from_numpy(np.random.default_rng(91).permutation(nb).astype(np.int64)).to(dev)
    pos = torch.arange(tokens, device=dev, dtype=torch.int64)
    slots = perm[pos // bs] * bs + pos % bs
    s = torch.cuda.current_stream()
    pa.kv_append(cache, k_new, v_new, slots, stream=s)
    torch.cuda.synchronize()
    pa.pa_timing_read(0)
    pa.pa_timing_enable(True)
    for _ in range(steps):
        pa.kv_append(cache, k_new, v_new, slots, stream=s)
    torch.cuda.synchronize()
    pa.pa_timing_enable(False)
    tot, cnt = pa.pa_timing_read(0)
    k_ms = tot / cnt
    # K and V: bf16 read, E4M3 written; slots; each (token, head)'s two scales
    byts = 2 * tokens * hkv * d * (2 + 1) + tokens * 8 + tokens * hkv * 2 * 4
    out = {"workload": label, "tokens": tokens, "kernel_ms": round(k_ms, 4),
           "GB/s": round(byts / (k_ms * 1e-3) / 1e9, 1),
           "frac": round(byts / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": int(byts)}
    del kc, vc, k_new, v_new
    torch.cuda.empty_cache()
    return out


def measure_peaks(pa, torch, dev):
    """The chip's practical ceilings, measured with the instructions the
    kernels use (the library's measurement hooks): back-to-back bf16 MFMAs on
    every CU, and a streaming read of 4 GiB through LDS with the decode
    kernels' non-temporal LDS-filling loads.
    Each runs ~0.2 s first so the clock has settled."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(launch, n):
        t0 = time.time()
        while time.time() - t0 < 0.2:
            launch()
            torch.cuda.synchronize()
        e0.record(s)
        for _ in range(n):
            launch()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    iters = 8192
    out = torch.empty(pa.PEAK_MFMA_THREADS, dtype=torch.float32, device=dev)
    ms_m = timed(lambda: pa.pa_peak_mfma(out, iters, stream=s), 20)
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    outr = torch.empty(pa.PEAK_READ_THREADS, dtype=torch.int32, device=dev)
    ms_r = timed(lambda: pa.pa_peak_read(buf, outr, stream=s), 10)
    res = {"mfma_bf16_TFLOP/s": round(pa.PEAK_MFMA_FLOPS_PER_ITER * iters / (ms_m * 1e-3) / 1e12, 1),
           "hbm_read_GB/s": round(buf.numel() / (ms_r * 1e-3) / 1e9, 1),
           "how": "bf16 16x16x32 MFMA loop, 8 waves per CU; 4 GiB streaming read through LDS "
                  "with the decode kernels' non-temporal LDS-filling loads; measured after the "
                  "workloads, ~0.2 s warm-up each"}
    del buf, out, outr
    torch.cuda.empty_cache()
    return res


def add_measured_fractions(obj, peaks):
    """Beside each roofline's fraction of the published peak, its fraction of
    the measured ceiling for the same resource."""
    if isinstance(obj, dict):
        rl = obj.get("roofline")
        if isinstance(rl, dict) and "achieved" in rl:
            ref = peaks["mfma_bf16_TFLOP/s"] if rl.get("bound") == "mfma" else peaks["hbm_read_GB/s"]
            rl["frac_of_measured"] = round(rl["achieved"] / ref, 4)
        for v in obj.values():
            add_measured_fractions(v, peaks)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(spec, budget_s, min_rows=512):
    """The oracle, as it stands, on a bounded sample of the workload's query rows
    (all heads), on this host's cores: at least min_rows rows (more if the
    budget allows), with the host's provenance and a one-thread rate on the
    tiny workload and on a few rows of this one.  Rate in the metric's unit."""
    import oracle
    import torch
    import workloads as W

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def prepared(sp):
        b = W.make_batch(sp, "cpu")
        kc, vc = bits(b.k_pool).copy(), bits(b.v_pool).copy()
        oracle.kv_append(kc, vc, None, None, oracle.KV_BF16, bits(b.k_new), bits(b.v_new),
                         b.slot_mapping.numpy())
        return b, kc, vc, bits(b.q)

    def timed_rows(b, kc, vc, q, sp, rows):
        t0 = time.time()
        oracle.attention(q, kc, vc, None, None, oracle.KV_BF16, b.block_tables, b.hist, b.incr,
                         sp.num_q_heads, sp.scale, rows=rows)
        dt = max(time.time() - t0, 1e-6)
        rs = np.concatenate([[0], np.cumsum(b.incr)])
        pairs = 0
        for r in rows:
            s = int(np.searchsorted(rs, r, side="right") - 1)
            pairs += int(b.hist[s]) + int(r - rs[s]) + 1
        return 4 * sp.head_dim * sp.num_q_heads * pairs / dt / 1e12, dt

    b, kc, vc, q = prepared(spec)
    rng = np.random.default_rng(0)
    n_incr = int(b.incr[0])
    # calibrate with a few rows, then size the sample to the budget (at least min_rows)
    _, t1 = timed_rows(b, kc, vc, q, spec, [n_incr - 1])
    n = int(max(min(min_rows, n_incr), min(n_incr, budget_s / t1)))
    rows = np.sort(rng.choice(n_incr, size=n, replace=False)).astype(np.int64)
    value, dt = timed_rows(b, kc, vc, q, spec, rows)
    threads = oracle.num_threads()
    # one thread: the tiny workload (all rows) and four rows of this one
    prev = oracle.set_num_threads(1)
    try:
        tb = prepared(W.tiny())
        tiny_1t, tiny_s = timed_rows(*tb, W.tiny(), list(range(W.tiny().total_q)))
        incr_1t, incr_s = timed_rows(b, kc, vc, q, spec, list(rows[:: max(1, len(rows) // 4)][:4]))
    finally:
        oracle.set_num_threads(prev)
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {n_incr} query rows (all {spec.num_q_heads} heads) of the headline "
                      f"workload, fp64, {dt:.1f} s on {threads} threads",
            "host": {"cpu_model": _cpu_model(), "nproc": len(os.sched_getaffinity(0)),
                     "os_cpu_count": os.cpu_count(), "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")},
            "one_thread": {"tiny_TFLOP/s": tiny_1t, "tiny_s": round(tiny_s, 3),
                           "incremental_TFLOP/s": incr_1t, "incremental_rows": 4,
                           "incremental_s": round(incr_s, 2)}}


# ---------------------------------------------------------------------------
# rocprofv3 summaries.  The commands below are run from /tmp with
# TMPDIR=/tmp and OUT an absolute output directory; --summarize-profiles OUT
# then writes the text summaries committed under profiles/.
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_CMDS = {
    "ktrace": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/ktrace -o kt -- "
              "python3 REPO/bench.py --steps 10 --warmup 2 --no-cpu",
    "ktrace_only": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/ktrace_{w} -o kt -- "
                   "python3 REPO/bench.py --only {w} --steps 10 --warmup 2",
    "pmc": "rocprofv3 --pmc {counter} --output-format csv -d OUT/pmc/{w}_{counter} -o p -- "
           "python3 REPO/bench.py --only {w} --steps 2 --warmup 1",
    "copy": "rocprofv3 --pmc {counter} --output-format csv -d OUT/pmc/copy_{counter} -o p -- "
            "python3 REPO/bench.py --copy-calibration 1024 --steps 2",
    "pmc_set": "rocprofv3 --pmc {counters} --output-format csv -d OUT/pmcx/{w}_{i} -o p -- "
               "python3 REPO/bench.py --only {w} --steps 2 --warmup 1",
}
# counter passes behind profiles/design_counters.txt (each within one pass's
# hardware limits: at most 8 SQ, 4 TCC, 2 GRBM counters)
DESIGN_COUNTER_SETS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVES "
                       "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE",
                       "TCC_HIT_sum TCC_MISS_sum"]
KERNEL_SOURCES = ["paged_kv_cache_gqa_amd/csrc/pa_attention.hip",
                  "paged_kv_cache_gqa_amd/csrc/pa_device.h",
                  "paged_kv_cache_gqa_amd/csrc/pa_internal.h",
                  "paged_kv_cache_gqa_amd/csrc/pa_append.hip",
                  "paged_kv_cache_gqa_amd/csrc/pa_api.hip"]  # the planner sets the access order
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
# (the prefill and append kernels' last template argument is the KV format:
# 0 bf16, 1 E4M3, 2 MXFP4)
PREFILL_KERNEL = "void pa::prefill_w48_kernel<16, 0>(pa::AttnArgs)"
PREFILL_FP8_KERNEL = "void pa::prefill_w48_kernel<64, 1>(pa::AttnArgs)"
PREFILL_FP4_KERNEL = "void pa::prefill_w48_kernel<64, 2>(pa::AttnArgs)"
DECODE_KERNEL = "void pa::decode_dma_kernel<16, 8, 2>(pa::AttnArgs)"
DECODE_CLAIM_KERNEL = ("void pa::decode_claim_kernel<16, 0, 0>(pa::AttnArgs, unsigned int*, int, pa::CascadeItem const*, "
                       "pa::CascadeMember const*, int)")
DECODE_FP8_KERNEL = "void pa::decode_dma_fp8_kernel<64, 8, 2>(pa::AttnArgs)"
DECODE_FP4_KERNEL = "void pa::decode_dma_fp4_kernel<64, 8, 2>(pa::AttnArgs)"
APPEND_KERNEL = "void pa::append_kernel<0>(pa::AppendArgs)"
# (--only workload, kernel, summary name, key in TRAFFIC_FILE)
PROFILED = [("incremental", PREFILL_KERNEL, "incremental_45.7k_to_48.4k", "prefill_incremental_bytes"),
            ("incremental_128k", PREFILL_KERNEL, "incremental_131k_to_133.8k", "prefill_incremental_128k_bytes"),
            ("decode", DECODE_KERNEL, "decode_batch_64x142k", "decode_batch_bytes"),
            ("long_decode", DECODE_FP8_KERNEL, "decode_e4m3_context_1m", "decode_long_e4m3_bytes"),
            ("long_decode_mxfp4", DECODE_FP4_KERNEL, "decode_mxfp4_context_1m", "decode_long_mxfp4_bytes"),
            ("long_prefill", PREFILL_FP8_KERNEL, "prefill_e4m3_1m_plus_4096", "prefill_long_e4m3_bytes"),
            ("long_prefill_mxfp4", PREFILL_FP4_KERNEL, "prefill_mxfp4_1m_plus_4096", "prefill_long_mxfp4_bytes"),
            ("kv_append_1m", APPEND_KERNEL, "kv_append_1m_bf16", "kv_append_1m_bytes"),
            ("mixed_sequential", PREFILL_KERNEL, "mixed_step_prefill_part", "prefill_mixed_bytes"),
            ("mixed_sequential", DECODE_KERNEL, "mixed_step_decode_part", "decode_mixed_bytes")]


def only_spec(W, name):
    """The workload of bench.py --only NAME."""
    return {"incremental": lambda: W.incremental(), "decode": lambda: W.decode_batch(),
            "incremental_128k": lambda: W.incremental(131_072, 2_700, "incremental_128k"),
            "long_decode": lambda: W.long_context(1_048_575, 1), "mixed": lambda: W.mixed(),
            "mixed_sequential": lambda: W.mixed(),
            "long_decode_mxfp4": lambda: W.long_context_mxfp4(1_048_575, 1),
            "long_prefill": lambda: W.long_context(), "long_prefill_mxfp4": lambda: W.long_context_mxfp4()}[name]()


def algorithmic_work(W, name, kernel=None):
    """(flops, bytes) of one launch of the profiled kernel of bench.py --only NAME."""
    if name == "kv_append_1m":
        return 0, 2 * 1_048_576 * 8 * 128 * 2 * 2 + 1_048_576 * 8
    spec = only_spec(W, name)
    if name in ("mixed", "mixed_sequential"):
        fl, dfl, byts = mixed_parts(spec)
        return (dfl, byts) if kernel == DECODE_KERNEL else (fl, 0)
    fl = prefill_flops(spec.hist, spec.incr, spec.num_q_heads, spec.head_dim)
    return fl, decode_bytes(spec) if name in ("decode", "long_decode", "long_decode_mxfp4") else prefill_bytes(spec)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def _counter_means(path):
    import csv
    import glob
    f = glob.glob(os.path.join(path, "*counter_collection.csv"))[0]
    acc = {}
    for r in csv.DictReader(open(f)):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _stats_table(fh, stats):
    fh.write("  Name | Calls | AverageNs | MinNs | MaxNs\n")
    for r in stats:
        if r["Name"].startswith(("void pa::", "pa::")):
            fh.write(f"  {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{r['MinNs']} | {r['MaxNs']}\n")


def summarize_profiles(out):
    import csv
    import glob
    def load(sub, what):
        return list(csv.DictReader(open(glob.glob(os.path.join(out, sub, f"*{what}.csv"))[0])))

    copy_f = _counter_means(os.path.join(out, "pmc", "copy_FETCH_SIZE"))["__amd_rocclr_copyBuffer"][0]
    copy_w = _counter_means(os.path.join(out, "pmc", "copy_WRITE_SIZE"))["__amd_rocclr_copyBuffer"][0]
    gib = float(1 << 30)
    f_scale, w_scale = gib / (copy_f * 1024), gib / (copy_w * 1024)
    src = kernel_source_hash()
    traffic = {}
    for w, kname, unit_desc, key in PROFILED:
        fetch, nf = _counter_means(os.path.join(out, "pmc", f"{w}_FETCH_SIZE"))[kname]
        write, nw = _counter_means(os.path.join(out, "pmc", f"{w}_WRITE_SIZE"))[kname]
        tb = fetch * 1024 * f_scale + write * 1024 * w_scale
        traffic[key] = tb
        stats = load(f"ktrace_{w}", "kernel_stats")
        st = {r["Name"]: r for r in stats}[kname]
        kshort = kname.split("pa::")[1].split("(")[0].replace("<", "_").replace(">", "").replace(", ", "_")
        fn = os.path.join(ROOT, "profiles", f"{kshort}__{unit_desc}.txt")
        with open(fn, "w") as fh:
            fh.write(f"Kernel: {kname}\nWorkload: {unit_desc} (bench.py --only {w})\n\n")
            fh.write("Commands (run from /tmp with TMPDIR=/tmp; OUT = output dir, REPO = repo root):\n")
            fh.write("  " + PROFILE_CMDS["ktrace_only"].format(w=w) + "\n")
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                fh.write("  " + PROFILE_CMDS["pmc"].format(counter=c, w=w) + "\n")
                fh.write("  " + PROFILE_CMDS["copy"].format(counter=c) + "\n")
            fh.write(f"  python3 REPO/bench.py --summarize-profiles OUT\n\n")
            fh.write("rocprofv3 --kernel-trace --stats (kernel_stats.csv rows of this run):\n")
            _stats_table(fh, stats)
            fh.write(f"\nThis kernel: average {float(st['AverageNs']) / 1e6:.4f} ms over {st['Calls']} calls\n")
            durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    for r in load(f"ktrace_{w}", "kernel_trace") if r["Kernel_Name"] == kname]
            timed = durs[-10:]  # the clean timed pass of 10 steps; earlier calls are warm-up and the instrumented pass
            fh.write(f"  timed steps only (last {len(timed)} dispatches, from kernel_trace.csv): "
                     f"average {sum(timed) / len(timed) / 1e6:.4f} ms\n\n")
            fh.write("HBM counters per dispatch (mean over dispatches of this kernel):\n")
            fh.write(f"  FETCH_SIZE {fetch:.1f} KiB ({nf} dispatches), WRITE_SIZE {write:.1f} KiB ({nw})\n")
            fh.write(f"  copy calibration (1 GiB device copy): FETCH_SIZE {copy_f:.1f} KiB, WRITE_SIZE {copy_w:.1f} KiB\n")
            fh.write(f"  scale factors: read x{f_scale:.4f}, write x{w_scale:.4f}\n")
            fh.write(f"  HBM traffic per launch = {tb / 1e9:.4f} GB\n")
            fh.write(f"\nKernel sources sha256[:16] = {src}\n")
    # every kernel of a default bench run (headline, decode, 128K and the reports)
    with open(os.path.join(ROOT, "profiles", "all_kernels__bench_default_run.txt"), "w") as fh:
        fh.write("All kernels of one bench.py run (headline, decode batch, 128K history and the\n"
                 "reports: initial prefill, 128K x 4,096, mixed step, 1M-token E4M3 prefill and\n"
                 "decode, kv_append); per-kernel averages mix the workloads that launch it.\n\n")
        fh.write("Command (run from /tmp with TMPDIR=/tmp; OUT = output dir, REPO = repo root):\n")
        fh.write("  " + PROFILE_CMDS["ktrace"] + "\n\n")
        _stats_table(fh, load("ktrace", "kernel_stats"))
        fh.write(f"\nKernel sources sha256[:16] = {src}\n")
    if os.path.isdir(os.path.join(out, "ktrace_mixed")):
        summarize_coscheduled(out, src)
    if os.path.isdir(os.path.join(out, "pmcx")):
        summarize_design_counters(out, src)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("# HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE, scaled by a 1 GiB copy\n")
        fh.write(f"source_hash={src}\n")
        for key, v in traffic.items():
            fh.write(f"{key}={v:.0f}\n")
    print(f"wrote profiles for source {src}")


def summarize_coscheduled(out, src):
    """profiles/decode_claim_kernel_16_0_0__mixed_step_coscheduled.txt: the
    mixed step as the planner runs it, from a kernel trace of bench.py --only
    mixed: per timed step, when the prefill and the two decode launches ran
    (the first beside the prefill on a second queue, the second after it)."""
    import csv
    import glob
    rows = list(csv.DictReader(open(glob.glob(os.path.join(out, "ktrace_mixed", "*kernel_trace.csv"))[0])))
    stats = list(csv.DictReader(open(glob.glob(os.path.join(out, "ktrace_mixed", "*kernel_stats.csv"))[0])))

    def t(r, k):
        return int(r[k + "_Timestamp"])

    pre = [r for r in rows if r["Kernel_Name"] == PREFILL_KERNEL][-10:]
    claims = [r for r in rows if r["Kernel_Name"] == DECODE_CLAIM_KERNEL]
    fn = os.path.join(ROOT, "profiles", "decode_claim_kernel_16_0_0__mixed_step_coscheduled.txt")
    with open(fn, "w") as fh:
        fh.write(f"Kernels: {PREFILL_KERNEL} and {DECODE_CLAIM_KERNEL}\n"
                 "Workload: mixed step, co-scheduled as the planner chooses (bench.py --only mixed)\n\n"
                 "Command (run from /tmp with TMPDIR=/tmp; OUT = output dir, REPO = repo root):\n"
                 "  " + PROFILE_CMDS["ktrace_only"].format(w="mixed") + "\n"
                 "  python3 REPO/bench.py --summarize-profiles OUT\n\n"
                 "rocprofv3 --kernel-trace --stats (kernel_stats.csv rows of this run):\n")
        _stats_table(fh, stats)
        fh.write("\nThe last 10 steps (kernel_trace.csv), ms from the prefill's start:\n"
                 "  prefill [start, end] (queue) | decode beside it [start, end] (queue) | "
                 "decode after it [start, end] | prefill start to last decode end\n")
        spans, pdur, bdur = [], [], []
        for p in pre:
            p0, p1 = t(p, "Start"), t(p, "End")
            beside = [c for c in claims if t(c, "Start") < p1 and t(c, "End") > p0]
            after = [c for c in claims if t(c, "Start") >= p1 and t(c, "Start") - p1 < 2_000_000]
            if not beside or not after:
                continue
            b, a = beside[0], after[0]

            def ms(x):
                return (x - p0) / 1e6

            end = max(p1, t(b, "End"), t(a, "End"))
            spans.append(ms(end))
            pdur.append(ms(p1))
            bdur.append((t(b, "End") - t(b, "Start")) / 1e6)
            fh.write(f"  [0, {ms(p1):.3f}] ({p['Queue_Id']}) | [{ms(t(b, 'Start')):.3f}, {ms(t(b, 'End')):.3f}] "
                     f"({b['Queue_Id']}) | [{ms(t(a, 'Start')):.3f}, {ms(t(a, 'End')):.3f}] | {ms(end):.3f}\n")
        if spans:
            fh.write(f"\nAverages over {len(spans)} steps: prefill {sum(pdur) / len(pdur):.3f} ms, decode beside "
                     f"it {sum(bdur) / len(bdur):.3f} ms, prefill start to last decode end "
                     f"{sum(spans) / len(spans):.3f} ms\n")
        fh.write(f"\nKernel sources sha256[:16] = {src}\n")


def summarize_design_counters(out, src):
    """profiles/design_counters.txt: the counters behind the design choices,
    per profiled kernel (mean over its dispatches)."""
    import csv
    import glob
    import workloads as W
    n_simd, n_xcc = 1024, 8
    with open(os.path.join(ROOT, "profiles", "design_counters.txt"), "w") as fh:
        fh.write("rocprofv3 counters behind the design choices (MI355X: 256 CUs, 1,024 SIMDs, 8 XCDs).\n"
                 "Commands (run from /tmp with TMPDIR=/tmp; OUT = output dir, REPO = repo root), per workload W:\n")
        for i, cs in enumerate(DESIGN_COUNTER_SETS):
            fh.write("  " + PROFILE_CMDS["pmc_set"].format(counters=cs, w="W", i=i) + "\n")
        fh.write("  python3 REPO/bench.py --summarize-profiles OUT\n"
                 "Derived: clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /\n"
                 "(GRBM_GUI_ACTIVE / 8 * 1,024 SIMDs); MFMA work / algorithmic = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 /\n"
                 "the workload's algorithmic flops (padding: the all-ones row-sum block, the last tile's\n"
                 "padded rows, the causal diagonal; decode packs G = 4 heads into 16 MFMA columns);\n"
                 "LDS conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS).\n\n")
        for w, kname, unit_desc, _ in PROFILED:
            vals, durs = {}, []
            for i in range(len(DESIGN_COUNTER_SETS)):
                fs = glob.glob(os.path.join(out, "pmcx", f"{w}_{i}", "*counter_collection.csv"))
                if not fs:
                    continue
                for r in csv.DictReader(open(fs[0])):
                    if r["Kernel_Name"] != kname:
                        continue
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    if i == 0 and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                        durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            if not vals:
                continue
            m = {k: sum(v) / len(v) for k, v in vals.items()}
            fl, byts = algorithmic_work(W, w, kname)
            fh.write(f"{kname} -- {unit_desc} (bench.py --only {w}), {len(durs)} dispatches\n")
            for k in sorted(m):
                fh.write(f"  {k:32s} {m[k]:.6g}\n")
            dur = sum(durs) / len(durs) * 1e-9 if durs else None
            gui = m.get("GRBM_GUI_ACTIVE", 0) / n_xcc
            if dur:
                fh.write(f"  duration (counter run)           {dur * 1e3:.4f} ms\n")
                fh.write(f"  clock                            {gui / dur / 1e9:.3f} GHz\n")
            if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                fh.write(f"  MFMA busy                        {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * n_simd):.3f}\n")
            if fl and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
                fh.write(f"  MFMA work / algorithmic flops    {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / fl:.3f}\n")
            if m.get("SQ_LDS_IDX_ACTIVE"):
                fh.write(f"  LDS conflict share               {m.get('SQ_LDS_BANK_CONFLICT', 0) / m['SQ_LDS_IDX_ACTIVE']:.4f}\n")
            if "TCC_HIT_sum" in m:
                fh.write(f"  L2 hit                           {m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.3f}\n")
            if dur:
                if fl:
                    fh.write(f"  algorithmic rate (counter run)   {fl / dur / 1e12:.1f} TFLOP/s\n")
                if byts:
                    fh.write(f"  algorithmic bytes / duration     {byts / dur / 1e9:.1f} GB/s\n")
            fh.write("\n")
        fh.write(f"Kernel sources sha256[:16] = {src}\n")


def measured_traffic(key):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    try:
        kv = dict(l.strip().split("=", 1) for l in open(TRAFFIC_FILE) if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash") != kernel_source_hash():
        return None
    return float(kv[key]) if key in kv else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-reports", action="store_true",
                    help="skip the other workloads (initial prefill, 128K x 4,096, mixed step, "
                         "1M-token E4M3 prefill and decode, kv_append bandwidth)")
    ap.add_argument("--no-128k", action="store_true",
                    help="skip the 128K-history incremental prefill (same kernel as the headline)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/*.txt from rocprofv3 outputs under DIR and exit")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA and HBM-read ceilings")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--only", choices=["incremental", "decode", "incremental_128k", "long_decode", "kv_append_1m",
                                       "mixed", "mixed_sequential", "long_decode_mxfp4", "long_prefill",
                                       "long_prefill_mxfp4"],
                    help="run one workload (for profiling); prints its JSON object")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(no sharding or collectives), so only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_gqa_amd as pa
    import workloads as W
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": max(1, args.steps)}))
        return
    if args.only == "kv_append_1m":
        print(json.dumps(report_append(pa, torch, dev, 1_048_576, max(1, args.steps),
                                       "kv_append of 1,048,576 bf16 tokens")))
        return
    if args.only:
        spec = only_spec(W, args.only)
        if args.only == "mixed_sequential":  # the prefill and decode launches one after the other
            pa.pa_debug_overlap_cus(0)
        r = Runner(pa, torch, spec, dev)
        ms, kern = r.timed(args.steps, args.warmup)
        print(json.dumps({"workload": args.only, "ms_per_step": round(ms, 4),
                          "kernels_ms": {k: round(v[0], 4) for k, v in kern.items()}}))
        return

    spec = W.incremental()
    r = Runner(pa, torch, spec, dev)
    ms, kern = r.timed(args.steps, args.warmup)
    flops = prefill_flops(spec.hist, spec.incr, spec.num_q_heads, spec.head_dim)
    value = flops / (ms * 1e-3) / 1e12
    k_ms = kern["prefill"][0]
    k_launch_per_step = kern["prefill"][1]
    achieved = flops / (k_ms * k_launch_per_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "incremental_prefill: 1 session, 45,700 cached + 2,700 new tokens, "
                               "32 q / 8 KV heads, head_dim 128, block 16, bf16 KV, one layer",
                   "hist": spec.hist[0], "incr": spec.incr[0], "num_q_heads": 32,
                   "num_kv_heads": 8, "head_dim": 128, "block_size": 16},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_incremental_bytes"),
                     "kernel": "prefill_w48_kernel<16, 0>",
                     "kernel_ms": round(k_ms, 4)},
        "kernels_ms": {k: round(v[0], 4) for k, v in kern.items()},
    }
    del r
    torch.cuda.empty_cache()

    if not args.no_extra:
        # batched decode, 64 sessions, median context 142K
        dspec = W.decode_batch()
        r = Runner(pa, torch, dspec, dev)
        dms, dk = r.timed(args.steps, args.warmup)
        byts = decode_bytes(dspec)
        dk_ms = dk["decode"][0]
        line["decode"] = {
            "workload": "decode_batch: 64 sessions x 1 token, lognormal context (median 142K, "
                        "sigma 0.5, clipped [10K, 256K]), 32 q / 8 KV heads, d 128, block 16, bf16",
            "sum_ctx": int(sum(dspec.hist) + 64),
            "ms_per_step": round(dms, 4),
            "GB/s": round(byts / (dms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(64 / (dms * 1e-3), 1),
            "kernels_ms": {k: round(v[0], 4) for k, v in dk.items()},
            "roofline": {"bound": "hbm", "achieved": round(byts / (dk_ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(byts / (dk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_batch_bytes"),
                         "algorithmic_bytes": int(byts), "kernel": "decode_dma_kernel<16, 8, 2>",
                         "kernel_ms": round(dk_ms, 4)},
        }
        del r
        torch.cuda.empty_cache()
    if not args.no_extra and not args.no_128k:
        # incremental prefill at 128K history
        pspec = W.incremental(131_072, 2_700, "incremental_128k")
        r = Runner(pa, torch, pspec, dev)
        pms, pk = r.timed(max(3, args.steps // 2), args.warmup)
        pfl = prefill_flops(pspec.hist, pspec.incr, 32, 128)
        pk_ms = pk["prefill"][0] * pk["prefill"][1]
        line["prefill_128k"] = {
            "workload": "incremental_prefill: 131,072 cached + 2,700 new tokens, 32 q / 8 KV, d 128",
            "ms_per_step": round(pms, 4), "TFLOP/s": round(pfl / (pms * 1e-3) / 1e12, 2),
            "kernels_ms": {k: round(v[0], 4) for k, v in pk.items()},
            "roofline": {"bound": "mfma", "achieved": round(pfl / (pk_ms * 1e-3) / 1e12, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pfl / (pk_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_incremental_128k_bytes"),
                         "kernel": "prefill_w48_kernel<16, 0>", "kernel_ms": round(pk_ms, 4)},
        }
        del r
        torch.cuda.empty_cache()

    if not args.no_extra and not args.no_reports:
        rs, rw = max(3, args.steps // 2), max(1, args.warmup)
        rep = {}
        rep["initial_prefill"] = report_prefill(
            pa, torch, W.initial(), dev, max(3, args.steps // 4), rw,
            "initial_prefill: 45,700 tokens, no history, 32 q / 8 KV heads, d 128, block 16, bf16")
        rep["incremental_128k_4096"] = report_prefill(
            pa, torch, W.incremental(131_072, 4_096, "incremental_128k_4096"), dev, rs, rw,
            "incremental_prefill: 131,072 cached + 4,096 new tokens, 32 q / 8 KV, d 128, bf16")
        rep["mixed_step"] = report_mixed(
            pa, torch, W.mixed(), dev, rs, rw,
            "mixed: 4 incremental prefills (lognormal histories, median 100K) + 48 decodes "
            "(8 over a shared 10,000-token prefix), 32 q / 8 KV, d 128, block 16, bf16, one call "
            "(the decode co-scheduled beside the prefill as the planner chooses)")
        rep["mixed_step_sequential"] = report_mixed(
            pa, torch, W.mixed(), dev, rs, rw,
            "the same mixed step with the prefill and decode launches one after the other",
            overlap=0)
        rep["mixed_step_cascade"] = report_mixed(
            pa, torch, W.mixed(), dev, rs, rw,
            "the same mixed step through paged_attn_forward_cascade, the 8 sub-agents declared as a "
            "group over their shared 10,000 tokens", cascade=True)
        rep["mixed_step_one_launch"] = report_mixed_one_launch(
            pa, torch, W.mixed(), dev, rs, rw,
            "the same mixed step through paged_attn_step: kv_append, both attention parts and the merges "
            "in one persistent launch with device-side task claiming")
        lspec = W.long_context()
        lr = Runner(pa, torch, lspec, dev)
        rep["long_context_prefill_e4m3"] = report_prefill(
            pa, torch, lspec, dev, max(3, args.steps // 4), rw,
            "long_context: 1,044,480 cached + 4,096 new tokens, E4M3 KV with per-(block, head) "
            "scales, block 64, 32 q / 8 KV, d 128", runner=lr)
        rep["long_context_decode_e4m3"] = report_decode_steps(
            pa, torch, lr, dev,
            "long_context: the 256 decode steps after the prefill (contexts 1,048,577 to "
            "1,048,832), each appending one token, E4M3 KV, block 64")
        del lr
        torch.cuda.empty_cache()
        fspec = W.long_context_mxfp4()
        fr = Runner(pa, torch, fspec, dev)
        rep["long_context_prefill_mxfp4"] = report_prefill(
            pa, torch, fspec, dev, max(3, args.steps // 4), rw,
            "the same session with 4-bit KV: OCP MXFP4 (E2M1 codes, one E8M0 scale per 32 elements "
            "of a token and head), block 64", runner=fr)
        rep["long_context_decode_mxfp4"] = report_decode_steps(
            pa, torch, fr, dev,
            "the 256 decode steps after that prefill, MXFP4 KV, block 64")
        del fr
        torch.cuda.empty_cache()
        rep["kv_append_45700"] = report_append(pa, torch, dev, 45_700, 20,
                                               "kv_append of 45,700 bf16 tokens (initial prefill)")
        rep["kv_append_1m"] = report_append(pa, torch, dev, 1_048_576, 5,
                                            "kv_append of 1,048,576 bf16 tokens")
        rep["kv_append_e4m3_4096"] = report_append_e4m3(
            pa, torch, dev, 4_096, 20,
            "kv_append of the long-context step's 4,096 tokens into the E4M3 cache (block 64, quantising)")
        line["reports"] = rep
    if not args.no_peaks:
        peaks = measure_peaks(pa, torch, dev)
        line["measured_peaks"] = peaks
        add_measured_fractions(line, peaks)
    if not args.no_cpu:
        line["cpu_baseline"] = run_cpu_baseline(spec, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
