#!/usr/bin/env python3
"""Throughput of Flash-LoRA-Attention on one MI355X.

Primary line (the JSON ``value``): paged decode of 16 requests over 4 shared
8192-token contexts (4 agents per context), LLaMA-3.1-8B attention shape
(H_q 32, H_kv 8, d 128), rank 16, bf16 storage / fp32 accumulation, one
attention layer.  One step = one ``lra_attn_decode`` call over one batch;
value = requests (= new tokens) per second.  The roofline object is for that
decode kernel (HBM bound): algorithmic bytes per launch / average launch time
from HIP events on the launch stream.

Extra legs in the same run (``extra``): chunked prefill with RoPE on the adapter
key term (512 new tokens over 16384, 4 agents; TFLOP/s vs bf16 MFMA peak),
paged decode over 32 shuffled contexts of 4k-64k tokens (GB/s vs HBM peak),
the LR-cache build of one 4096-token layer (GB/s), and one whole PreLRShared
step (32 layers x (LR build + 8 agents' prefill of 4096 over 131072), TFLOP/s).

cpu_baseline: the float64 oracle on the host cores, on the primary workload's
first input set (all 16 requests, repeated until >= 10 s), as requests/s.

Inputs of sets that fit the 256 MB Infinity Cache are rotated over several
independent buffer sets so timed calls read HBM, not the cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + HBM GB/s % peak; prefill TFLOP/s % MFMA peak (1 GPU)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


# ----------------------------------------------------------------------------- accounting

def decode_bytes(ctx_len, n_req, n_agents_used, h_q, h_kv, d, r, esz=2, page=16):
    """Algorithmic HBM bytes of one decode call.

    Every context's base K/V (H_kv*d each) and shared LR rows (r each for L_k
    and L_v) are read once — the agents of a context share them — plus the
    queries, the referenced agents' B_k/B_v, the outputs and the index arrays
    (block-table entries in use, lengths, request offsets, agent ids).
    """
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    kv = int(ctx_len.sum()) * (2 * h_kv * d + 2 * r) * esz
    q = n_req * h_q * d * esz
    o = n_req * h_q * d * esz
    b = n_agents_used * 2 * r * h_kv * d * esz
    idx = int(((ctx_len + page - 1) // page).sum()) * 4 + len(ctx_len) * 4 + (len(ctx_len) + 1) * 4 \
        + n_req * 4
    return kv + q + o + b + idx


def decode_bytes_unshared(ctx_len_per_req, h_q, h_kv, d, r, esz=2):
    """Bytes if every request streamed its own full cache (no sharing): context only."""
    return int(np.sum(ctx_len_per_req)) * (2 * h_kv * d + 2 * r) * esz


def prefill_flops(n_req, q_len, kv_len, h_q, h_kv, d, r, rope):
    """Algorithmic flops of one prefill call (causal-masked work not credited).

    Per unmasked (row, key) pair: 4d (scores and values at head dimension) plus
    the rank-r terms: 2r on the value side (P L_v) and, without RoPE, 2r on the
    score side (qB . l_k).  With RoPE the adapter key is rebuilt at head
    dimension instead: 2 r d per (key, KV head, request).  Per query row: 2 r d
    for the single B_v post-multiplication, and without RoPE 2 r d for qB.
    """
    pairs = q_len * (kv_len - q_len) + q_len * (q_len + 1) // 2
    rows = n_req * q_len * h_q
    total = n_req * h_q * pairs * (4 * d + (2 * r if rope else 4 * r))
    total += rows * 2 * r * d * (1 if rope else 2)
    if rope:
        total += kv_len * h_kv * n_req * 2 * r * d
    return total


def lr_build_bytes(n_tok, d_model, r, esz=2):
    return (n_tok * d_model + 2 * r * d_model + 2 * n_tok * r) * esz


# ----------------------------------------------------------------------------- helpers

def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to("cuda")
    return torch.from_numpy(a).to("cuda")


def _randn_bf16(shape, sigma, gen):
    import torch
    x = torch.randn(shape, dtype=torch.float32, device="cuda", generator=gen)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def _time_calls(fn, n_sets, steps, warmup):
    """Average time per call (ms) over `steps` calls, HIP events on the launch stream."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i % n_sets)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def _call_stats(fn, n_sets, n_calls):
    """Per-call times (us) of n_calls back-to-back calls, one HIP event pair per call on the
    launch stream: median, p10, p90 (after the timed region, so it does not perturb it)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_calls)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i % n_sets)
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "calls": n_calls}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16__decode_4ctx_x_8192_r16__hbm_traffic.txt")
TRAFFIC_SOURCES = ("attention_shared_base_amd/csrc/decode_kernel.h", "attention_shared_base_amd/csrc/decode_bf16.hip",
                   "attention_shared_base_amd/csrc/api.hip")


def measured_traffic():
    """HBM bytes per launch of the primary decode kernel from the committed counter
    summary, or None if the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for src in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest()[:16] != kv.get("source_sha256"):
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- legs

class DecodeSet:
    def __init__(self, case):
        import workloads as w
        k, v, lk, lv = w.decode_device_layout(case.k_pool, case.v_pool, case.lk_pool, case.lv_pool)
        self.q, self.k, self.v, self.lk, self.lv = map(_dev, (case.q, k, v, lk, lv))
        self.crs = _dev(case.ctx_req_start())
        self.agent = _dev(case.req_agent)
        self.bt = _dev(case.block_table)
        self.clen = _dev(case.ctx_len)
        self.b_k, self.b_v = _dev(case.b_k), _dev(case.b_v)
        self.out = None


def primary_decode(steps, warmup, n_sets, rope_theta=None, per_agent=False, stats=None, rank=16):
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    if rank == 16:
        cases = [w.config2(layer=i) for i in range(n_sets)]
    else:  # the same shapes and draws at another rank
        cases = [w.make_decode(2, dtype="bf16", ctx_lens=[8192] * 4, reqs=[(b // 4, b % 4) for b in range(16)],
                               n_agents=4, h_q=32, h_kv=8, d=128, r=rank, shuffle=False, layer=i)
                 for i in range(n_sets)]
    sets = [DecodeSet(c) for c in cases]
    c0 = cases[0]
    mrpc = int(np.bincount(c0.req_ctx).max())
    max_len = int(c0.ctx_len.max())
    ws = torch.zeros(lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=rank, dtype=1, n_req=c0.n_req,
        n_ctx=c0.n_ctx, max_req_per_ctx=mrpc, max_ctx_len=max_len,
        lr_agent_stride=1 if per_agent else 0), dtype=torch.uint8, device="cuda")
    for s in sets:
        s.out = torch.empty_like(s.q)
        if per_agent:
            # one LR cache per agent (BaseShared): the agents' pools, own draws
            g = torch.Generator(device="cuda")
            g.manual_seed(11)
            n_ag = s.b_k.shape[0]
            s.lk = _randn_bf16((n_ag,) + tuple(s.lk.shape), 1.0, g)
            s.lv = _randn_bf16((n_ag,) + tuple(s.lv.shape), 1.0, g)
    cos = sin = None
    if rope_theta is not None:
        cos, sin = lra.rope_table(rope_theta, 128, max_len)

    def call(i):
        s = sets[i]
        lra.decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                   max_req_per_ctx=mrpc, max_ctx_len=max_len, rope_cos=cos, rope_sin=sin,
                   out=s.out, workspace=ws)

    ms = _time_calls(call, n_sets, steps, warmup)
    if stats is not None:
        stats.update(_call_stats(call, n_sets, max(20, min(steps, 200))))
    nbytes = decode_bytes(c0.ctx_len, c0.n_req, len(np.unique(c0.req_agent)), 32, 8, 128, rank)
    if rope_theta is not None:
        nbytes += 2 * max_len * 64 * 4  # the cos / sin rows, read once
    if per_agent:  # every agent of a context reads its own L_k, L_v rows
        n_ag_ctx = len(np.unique(c0.req_agent[c0.req_ctx == 0]))
        nbytes += int(c0.ctx_len.sum()) * 2 * rank * 2 * (n_ag_ctx - 1)
    return cases[0], ms, nbytes


def extra_workload1_fp32(steps, warmup):
    """The fp32 parity workload (2 agents over one 256-token context, Hq4 Hkv2 d64 r8): call time
    of its decode (2 requests) and its causal prefill (2 x 16 new tokens).  Launch-latency bound
    (a 278 KB working set); reported as time only."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    dec, pre = w.config1()
    s = DecodeSet(dec)
    d_out = torch.empty_like(s.q)
    q, agent = _dev(pre.q), _dev(pre.req_agent)
    k, v, lk, lv, bk, bv = map(_dev, (pre.k_base, pre.v_base, pre.l_k, pre.l_v, pre.b_k, pre.b_v))
    p_out = torch.empty_like(q)

    def call_d(_):
        lra.decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                   max_req_per_ctx=2, max_ctx_len=256, out=d_out)

    def call_p(_):
        lra.prefill(q, agent, k, v, lk, lv, bk, bv, out=p_out)

    ms_d = _time_calls(call_d, 1, steps, warmup)
    ms_p = _time_calls(call_p, 1, steps, warmup)
    return {"workload": "fp32 parity workload: 2 agents over one 256-token context (240 + 16 new), "
                        "Hq4 Hkv2 d64 r8; decode of 2 requests and prefill of 2 x 16 tokens",
            "value": ms_d * 1e3, "unit": "us per decode call", "ms_per_call": ms_d,
            "prefill_us_per_call": ms_p * 1e3,
            "roofline": None,
            "note": "launch-latency bound (278 KB working set): time only, no roofline"}


def extra_paged_decode(steps, warmup):
    """32 contexts of U[4096, 65536] tokens, shuffled 16-token pages, r 32 (5+ GB)."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    lens = w.config4_lengths()
    table, n_pages = w.page_table(4, lens, shuffle=True, max_blocks=65536 // 16)
    h_q, h_kv, d, r, n_req = 32, 8, 128, 32, 32
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    k = _randn_bf16((n_pages, h_kv, d // 8, 16, 8), 1.0, g)
    v = _randn_bf16((n_pages, h_kv, d, 16), 1.0, g)
    lk = _randn_bf16((n_pages, 16, r), 1.0, g)
    lv = _randn_bf16((n_pages, r, 16), 1.0, g)
    q = _randn_bf16((n_req, h_q, d), 1.0, g)
    b_k = _randn_bf16((8, r, h_kv * d), 0.05, g)
    b_v = _randn_bf16((8, r, h_kv * d), 0.05, g)
    crs = _dev(np.arange(33, dtype=np.int32))
    agent = _dev((np.arange(32) % 8).astype(np.int32))
    bt, clen = _dev(table), _dev(lens.astype(np.int32))
    out = torch.empty_like(q)
    max_len = int(lens.max())
    ws = torch.zeros(lra.decode_workspace_size(
        n_q_heads=h_q, n_kv_heads=h_kv, head_dim=d, rank=r, dtype=1, n_req=n_req, n_ctx=32,
        max_req_per_ctx=1, max_ctx_len=max_len), dtype=torch.uint8, device="cuda")

    def call(_):
        lra.decode(q, crs, agent, k, v, lk, lv, bt, clen, b_k, b_v, max_req_per_ctx=1,
                   max_ctx_len=max_len, out=out, workspace=ws)

    ms = _time_calls(call, 1, steps, warmup)
    nbytes = decode_bytes(lens, n_req, 8, h_q, h_kv, d, r)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "paged decode: 32 contexts of U[4096,65536] tokens (sum %d), shuffled "
                        "16-token pages, 32 requests over 8 agents, Hq32 Hkv8 d128 r32, bf16"
                        % int(lens.sum()),
            "value": n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None},
            "algorithmic_bytes": nbytes}


def extra_decode_rope(steps, warmup, base_ms):
    """The primary decode workload with RoPE (theta 5e5) on the adapter key term: each
    request's key adapter is rebuilt at head dimension and rotated per page."""
    case, ms, nbytes = primary_decode(steps, warmup, 4, rope_theta=500000.0)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "decode with RoPE on the adapter key: 16 requests over 4 shared 8192-token "
                    "contexts, Hq32 Hkv8 d128 r16, theta 5e5, bf16",
        "value": case.n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
        "time_vs_no_rope": ms / base_ms,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "algorithmic_bytes": nbytes,
    }


def extra_decode_qkvo_r4(steps, warmup):
    """The pages' query/key/value/output LoRA setting (LRAgent App. D.1): rank 4 with RoPE on
    the adapter key, against the plain rank-4 call on the same shapes (the cost of the key
    rebuild at the pages' rank)."""
    _, ms_plain, _ = primary_decode(steps, warmup, 4, rank=4)
    case, ms, nbytes = primary_decode(steps, warmup, 4, rope_theta=500000.0, rank=4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "decode, rank-4 LoRA with RoPE on the adapter key (qkvo setting): 16 requests "
                    "over 4 shared 8192-token contexts, Hq32 Hkv8 d128 r4, theta 5e5, bf16",
        "value": case.n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
        "ms_per_call_without_rope": ms_plain, "time_vs_no_rope": ms / ms_plain,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "algorithmic_bytes": nbytes,
    }


def extra_decode_per_agent(steps, warmup, base_ms):
    """The primary decode workload with one LR cache per agent (BaseShared / PreLRShared with
    per-agent A): each request reads its agent's L_k, L_v pages beside the shared base pages."""
    case, ms, nbytes = primary_decode(steps, warmup, 4, per_agent=True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "decode with one LR cache per agent: 16 requests over 4 shared 8192-token "
                    "contexts (4 agents each), Hq32 Hkv8 d128 r16, bf16",
        "value": case.n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
        "time_vs_shared_lr": ms / base_ms,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "algorithmic_bytes": nbytes,
    }


def extra_naive_decode(steps, warmup, base_ms):
    """Baseline of the Flash-LoRA comparison on the primary decode workload: every
    request's K, V materialised at head dimension (expansion kernel), then plain decode
    attention over the per-request caches.  Reported next to the method's time."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    n_sets = 2
    cases = [w.config2(layer=i) for i in range(n_sets)]
    sets = [DecodeSet(c) for c in cases]
    c0 = cases[0]
    mrpc = int(np.bincount(c0.req_ctx).max())
    max_len = int(c0.ctx_len.max())
    scratch = {}

    def call(i):
        s = sets[i]
        lra.naive_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                         max_req_per_ctx=mrpc, max_ctx_len=max_len, scratch=scratch)

    ms = _time_calls(call, n_sets, steps, warmup)
    n_tok = int(c0.ctx_len[c0.req_ctx].sum())
    # bytes the baseline moves: base K, V read and the expanded K, V written per request,
    # the expanded K, V read again by the attention (per KV head, bf16)
    kv_req = n_tok * 8 * 128 * 2 * 2
    nbytes = 3 * kv_req
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "baseline without Flash-LoRA-Attention: primary decode workload with each "
                    "request's K = K_base + L_k B_k, V = V_base + L_v B_v written to HBM, then "
                    "plain decode attention over the per-request caches",
        "value": c0.n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms,
        "method_speedup": ms / base_ms,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "algorithmic_bytes": nbytes,
    }


def extra_agent_scaling(steps, warmup):
    """Cross-agent cache sharing: the primary workload's 4 shared 8192-token contexts (two
    rotated sets of caches) decoded by 1, 2, 4, 8 and 16 requests per context, each with its own
    agent (B_k, B_v), beside the naive baseline that materialises every request's caches.  A row
    group holds 16 query rows (4 requests at 4 query heads per KV head): up to 4 agents per context
    every K/V page is read once, beyond that once per row group."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    sets = [DecodeSet(w.config2(layer=i)) for i in range(2)]
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    n_ag = 16
    b_k = _randn_bf16((n_ag, 16, 8 * 128), 0.05, g)
    b_v = _randn_bf16((n_ag, 16, 8 * 128), 0.05, g)
    table = {}
    for rpc in (1, 2, 4, 8, 16):
        n_req = 4 * rpc
        qs = [_randn_bf16((n_req, 32, 128), 1.0, g) for _ in sets]
        crs = torch.arange(0, n_req + 1, rpc, dtype=torch.int32, device="cuda")
        agent = torch.arange(n_req, dtype=torch.int32, device="cuda") % rpc
        out = torch.empty((n_req, 32, 128), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(16, lra.decode_workspace_size(
            n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1, n_req=n_req, n_ctx=4,
            max_req_per_ctx=rpc, max_ctx_len=8192)), dtype=torch.uint8, device="cuda")
        scratch = {}

        def call(i):
            st = sets[i]
            lra.decode(qs[i], crs, agent, st.k, st.v, st.lk, st.lv, st.bt, st.clen, b_k, b_v,
                       max_req_per_ctx=rpc, max_ctx_len=8192, out=out, workspace=ws)

        def call_naive(i):
            st = sets[i]
            lra.naive_decode(qs[i], crs, agent, st.k, st.v, st.lk, st.lv, st.bt, st.clen, b_k, b_v,
                             max_req_per_ctx=rpc, max_ctx_len=8192, scratch=scratch)

        ms = _time_calls(call, len(sets), steps, warmup)
        ms_naive = _time_calls(call_naive, len(sets), max(4, steps // 20), 2)
        table[str(rpc)] = {"decode_us": ms * 1e3, "naive_us": ms_naive * 1e3,
                           "decode_tokens_per_s": n_req / (ms * 1e-3)}
        del scratch, ws
        torch.cuda.empty_cache()
    t1, t4, t16 = (table[k]["decode_us"] for k in ("1", "4", "16"))
    return {"workload": "decode over 4 shared 8192-token contexts, Hq32 Hkv8 d128 r16, with 1, 2, 4, "
                        "8, 16 requests (agents) per context; method and naive materialising baseline",
            "value": t4 / t1, "unit": "x (time at 4 agents per context / time at 1)",
            "time_16_vs_1": t16 / t1, "per_agents": table, "roofline": None,
            "note": "scaling study: sharing the base and LR caches across agents"}


def extra_prefill_rope(steps, warmup, n_sets=2):
    """512 new tokens over a 16384-token shared context, 4 agents, RoPE 5e5 on the adapter key."""
    import torch
    import attention_shared_base_amd as lra
    n_req, q_len, kv_len, h_q, h_kv, d, r = 4, 512, 16896, 32, 8, 128, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    sets = []
    for _ in range(n_sets):
        sets.append(dict(
            q=_randn_bf16((n_req, q_len, h_q, d), 1.0, g),
            k=_randn_bf16((h_kv, kv_len, d), 1.0, g), v=_randn_bf16((h_kv, kv_len, d), 1.0, g),
            lk=_randn_bf16((kv_len, r), 1.0, g), lv=_randn_bf16((kv_len, r), 1.0, g),
            bk=_randn_bf16((4, r, h_kv * d), 0.05, g), bv=_randn_bf16((4, r, h_kv * d), 0.05, g)))
    agent = _dev(np.arange(4, dtype=np.int32))
    cos, sin = lra.rope_table(500000.0, d, kv_len)
    for s in sets:
        s["out"] = torch.empty_like(s["q"])

    def call(i):
        s = sets[i]
        lra.prefill(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bk"], s["bv"],
                    rope_cos=cos, rope_sin=sin, out=s["out"])

    ms = _time_calls(call, n_sets, steps, warmup)
    fl = prefill_flops(n_req, q_len, kv_len, h_q, h_kv, d, r, rope=True)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "chunked prefill: 512 new tokens over 16384 shared, 4 agents, RoPE "
                        "theta 5e5 on the adapter key term, Hq32 Hkv8 d128 r16, bf16",
            "value": tf, "unit": "TFLOP/s", "ms_per_call": ms,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS, "traffic": None},
            "algorithmic_flops": fl}


def extra_prefill_paged(steps, warmup, base_ms):
    """The prefill leg's workload with the context in shuffled 16-token pages
    (lra_attn_prefill_paged: staging of the context's rows, then the prefill)."""
    import torch
    import attention_shared_base_amd as lra
    n_req, q_len, kv_len, h_q, h_kv, d, r = 4, 512, 16896, 32, 8, 128, 16
    n_pages = kv_len // 16
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    sets = []
    for _ in range(2):
        sets.append(dict(
            q=_randn_bf16((n_req, q_len, h_q, d), 1.0, g),
            k=_randn_bf16((n_pages, h_kv, d // 8, 16, 8), 1.0, g),
            v=_randn_bf16((n_pages, h_kv, d, 16), 1.0, g),
            lk=_randn_bf16((n_pages, 16, r), 1.0, g), lv=_randn_bf16((n_pages, r, 16), 1.0, g),
            bk=_randn_bf16((4, r, h_kv * d), 0.05, g), bv=_randn_bf16((4, r, h_kv * d), 0.05, g),
            bt=torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32)))
    agent = _dev(np.arange(4, dtype=np.int32))
    cos, sin = lra.rope_table(500000.0, d, kv_len)
    ws = torch.empty(lra.prefill_paged_workspace_size(n_q_heads=h_q, n_kv_heads=h_kv, head_dim=d,
                                                      rank=r, kv_len=kv_len),
                     dtype=torch.uint8, device="cuda")
    for s in sets:
        s["out"] = torch.empty_like(s["q"])

    def call(i):
        s = sets[i]
        lra.prefill_paged(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bt"], kv_len,
                          s["bk"], s["bv"], rope_cos=cos, rope_sin=sin, out=s["out"], workspace=ws)

    ms = _time_calls(call, 2, steps, warmup)
    fl = prefill_flops(n_req, q_len, kv_len, h_q, h_kv, d, r, rope=True)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "paged chunked prefill: the prefill leg's workload (512 new tokens over "
                        "16384, 4 agents, RoPE) with the context in shuffled 16-token pages",
            "value": tf, "unit": "TFLOP/s", "ms_per_call": ms,
            "time_vs_contiguous": ms / base_ms if base_ms else None,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS, "traffic": None},
            "algorithmic_flops": fl}


def extra_lr_build(steps, warmup, n_sets=8):
    import torch
    import attention_shared_base_amd as lra
    n_tok, d_model, r = 4096, 4096, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    sets = [dict(x=_randn_bf16((n_tok, d_model), 1.0, g),
                 ak=_randn_bf16((r, d_model), 1.0 / 64, g), av=_randn_bf16((r, d_model), 1.0 / 64, g),
                 lk=torch.empty((n_tok, r), dtype=torch.bfloat16, device="cuda"),
                 lv=torch.empty((n_tok, r), dtype=torch.bfloat16, device="cuda"))
            for _ in range(n_sets)]
    # one zero-filled workspace for every call (the calls leave it ready)
    n_ws = lra.lr_cache_build_workspace_size(dtype=1, n_tok=n_tok, d_model=d_model, rank=r)
    ws = torch.zeros(max(n_ws, 16), dtype=torch.uint8, device="cuda")

    def call(i):
        s = sets[i]
        lra.lr_cache_build(s["x"], s["ak"], s["av"], s["lk"], s["lv"], workspace=ws)

    ms = _time_calls(call, n_sets, steps, warmup)
    nbytes = lr_build_bytes(n_tok, d_model, r)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "LR-cache build L = X [A_k|A_v]: X [4096, 4096] bf16, r 16",
            "value": gbs, "unit": "GB/s", "ms_per_call": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None},
            "algorithmic_bytes": nbytes}


def extra_prelr_step(steps, warmup, n_layers=32):
    """PreLRShared step: per layer, LR build of 4096 new rows, then 8 agents' prefill.

    32 layers of LLaMA-3.1-8B attention shape, each with its own buffers: X
    [4096, 4096], A_k/A_v [16, 4096], K_base/V_base [8, 135168, 128] (131072
    old + 4096 new tokens), L_k/L_v [135168, 16] (old rows given, new rows built
    in the step), per-agent Q [4096, 32, 128] and B [16, 1024].  Inputs are
    drawn on the GPU (torch Philox) with the same distributions as the seeded
    host generator; parity of this workload is covered by the tests.
    """
    import torch
    import attention_shared_base_amd as lra
    n_new, n_old, d_model, h_q, h_kv, d, r, n_ag = 4096, 131072, 4096, 32, 8, 128, 16, 8
    kv_len = n_old + n_new
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    layers = []
    for _ in range(n_layers):
        lk = _randn_bf16((kv_len, r), 1.0, gen)
        lv = _randn_bf16((kv_len, r), 1.0, gen)
        layers.append(dict(
            x=_randn_bf16((n_new, d_model), 1.0, gen),
            ak=_randn_bf16((r, d_model), 1.0 / 64, gen), av=_randn_bf16((r, d_model), 1.0 / 64, gen),
            k=_randn_bf16((h_kv, kv_len, d), 1.0, gen), v=_randn_bf16((h_kv, kv_len, d), 1.0, gen),
            lk=lk, lv=lv, q=_randn_bf16((n_ag, n_new, h_q, d), 1.0, gen),
            bk=_randn_bf16((n_ag, r, h_kv * d), 0.05, gen),
            bv=_randn_bf16((n_ag, r, h_kv * d), 0.05, gen)))
    agent = torch.arange(n_ag, dtype=torch.int32, device="cuda")
    out = torch.empty((n_ag, n_new, h_q, d), dtype=torch.bfloat16, device="cuda")
    n_ws = lra.lr_cache_build_workspace_size(dtype=1, n_tok=n_new, d_model=d_model, rank=r)
    ws = torch.zeros(max(n_ws, 16), dtype=torch.uint8, device="cuda")

    def call(_):
        for L in layers:
            lra.lr_cache_build(L["x"], L["ak"], L["av"], L["lk"], L["lv"], row_offset=n_old,
                               workspace=ws)
            lra.prefill(L["q"], agent, L["k"], L["v"], L["lk"], L["lv"], L["bk"], L["bv"], out=out)

    ms = _time_calls(call, 1, steps, warmup)
    fl = n_layers * (prefill_flops(n_ag, n_new, kv_len, h_q, h_kv, d, r, rope=False)
                     + 2 * n_new * d_model * 2 * r)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": "PreLRShared step: 32 layers x (LR build X[4096,4096]·[A_k|A_v] r16, then "
                        "8 agents' prefill of 4096 new tokens over 131072 shared), Hq32 Hkv8 d128, bf16",
            "value": tf, "unit": "TFLOP/s", "ms_per_call": ms,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS, "traffic": None},
            "algorithmic_flops": fl}


def copy_calibration(nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": nbytes, "launches": reps}), flush=True)


def cpu_baseline(case, min_seconds=10.0):
    """The float64 oracle, as it stands, on the primary workload's first input set."""
    import oracle
    import workloads as w
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    args = [w.widen(x) for x in (case.q, case.k_pool, case.v_pool, case.lk_pool, case.lv_pool,
                                 case.b_k, case.b_v)]
    q, kp, vp, lkp, lvp, bk, bv = args
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_paged(q, case.req_ctx, case.req_agent, kp, vp, lkp, lvp, case.block_table,
                            case.ctx_len, bk, bv)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": reps * case.n_req / el, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full decode call of the primary workload (16 requests x 8192 keys), "
                      f"repeated {reps}x in {el:.1f} s, float64 NumPy"}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets of the primary leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra legs")
    ap.add_argument("--extra", default="workload1_fp32,agent_scaling,decode_rope,decode_qkvo_r4,decode_per_agent,naive_decode,prefill_rope,"
                                       "prefill_paged,paged_decode,lr_build,prelr_step",
                    help="comma-separated extra legs to run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_shared_base_amd as lra
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    lra.load()

    _log("primary: decode, 4 shared contexts x 8192 tokens, 16 requests")
    call_us = {}
    case, ms, nbytes = primary_decode(args.steps, args.warmup, args.sets, stats=call_us)
    gbs = nbytes / (ms * 1e-3) / 1e9
    value = case.n_req / (ms * 1e-3)
    _log(f"primary: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s, {value:.0f} tokens/s")

    extra = {}
    if not args.no_extra:
        legs = {"decode_rope": lambda: extra_decode_rope(args.steps, args.warmup, ms),
                "decode_per_agent": lambda: extra_decode_per_agent(args.steps, args.warmup, ms),
                "decode_qkvo_r4": lambda: extra_decode_qkvo_r4(args.steps, args.warmup),
                "naive_decode": lambda: extra_naive_decode(max(5, args.steps // 10), 3, ms),
                "prefill_rope": lambda: extra_prefill_rope(max(5, args.steps // 10), 3),
                "prefill_paged": lambda: extra_prefill_paged(
                    max(5, args.steps // 10), 3,
                    extra.get("prefill_rope", {}).get("ms_per_call")),
                "paged_decode": lambda: extra_paged_decode(max(5, args.steps // 10), 3),
                "workload1_fp32": lambda: extra_workload1_fp32(args.steps, 10),
                "agent_scaling": lambda: extra_agent_scaling(max(20, args.steps // 2), 5),
                "lr_build": lambda: extra_lr_build(args.steps, 10),
                "prelr_step": lambda: extra_prelr_step(1, 1)}
        for name in [x for x in args.extra.split(",") if x]:
            fn = legs[name]
            _log(f"extra: {name}")
            try:
                extra[name] = fn()
                rl = extra[name].get("roofline")
                _log(f"extra: {name}: {extra[name]['value']:.4g} {extra[name]['unit']}"
                     + (f", {rl['frac'] * 100:.1f}% of peak" if rl else ""))
            except lra.LraError as e:
                extra[name] = {"error": str(e)}
                _log(f"extra: {name}: {e}")
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        _log("cpu baseline: oracle")
        cpu = cpu_baseline(case)

    unshared = decode_bytes_unshared(case.ctx_len[case.req_ctx], 32, 8, 128, 16)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) caches/queries, B ~ N(0,0.05^2)); no weights or datasets",
        "config": {
            "workload": "decode: 16 requests over 4 shared 8192-token contexts (4 agents per "
                        "context), Hq32 Hkv8 d128 r16, bf16 storage / fp32 accumulation, one "
                        "attention layer, 16-token pages",
            "input_sets_rotated": args.sets,
            "algorithmic_bytes_per_call": nbytes,
            "bytes_if_agents_did_not_share": unshared,
        },
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "call_us": call_us,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
