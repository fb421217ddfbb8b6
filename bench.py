#!/usr/bin/env python3
"""Throughput of Flash-LoRA-Attention on one MI355X.

Primary line (the JSON ``value``): paged decode of 16 requests over 4 shared
8192-token contexts (4 agents per context), LLaMA-3.1-8B attention shape
(H_q 32, H_kv 8, d 128), rank 16, bf16 storage / fp32 accumulation, one
attention layer.  One step = one ``lra_attn_decode`` call over one batch;
value = requests (= new tokens) per second.  The roofline object is for that
decode kernel (HBM bound): algorithmic bytes per launch / average launch time
from HIP events on the launch stream.

Extra legs in the same run (``extra``), each with its roofline, per-call
median / p10 / p90, the float64 oracle timed on the host cores
(``cpu_baseline``) and a parity check of the timed outputs against the oracle:
the fp32 parity workload, decode variants (RoPE on the adapter key, the rank-4
qkvo setting, one LR cache per agent, the naive materialising baseline, the
cross-agent sharing sweep), chunked prefill with RoPE (512 new tokens over
16384, 4 agents) from contiguous caches and from shuffled pages, paged decode
over 32 shuffled contexts of 4k-64k tokens, the LR-cache build of one 4096-token
layer, and one whole PreLRShared step (32 layers x (LR build + 8 agents'
prefill of 4096 over 131072)).

Inputs of sets that fit the 256 MB Infinity Cache are rotated over several
independent buffer sets (>= 512 MB together) so timed calls read HBM.
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
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
BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS = 2e-2, 1e-2, 1e-5
# False (--no-oracle, for profiling runs): legs skip the oracle timing and parity
CHECK = True
UNCHECKED = {"cpu_baseline": None, "parity": None, "note_oracle": "oracle not run (--no-oracle)"}


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
    return torch.from_numpy(a).to("cuda")


def _host(t):
    """Device tensor -> float64 numpy (exact widening of bf16 / fp32)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def _randn_bf16(shape, sigma, gen):
    import torch
    x = torch.randn(shape, dtype=torch.float32, device="cuda", generator=gen)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


# Extra legs time a kernel only after at least this much of its own calls: the chip runs
# the first tens of milliseconds of a new heavy kernel slower (workload-3 prefill: about
# 800 us per call falling to 650 us over its first 40 calls, with or without other load
# before it), so a short warm-up would time that transient instead of the steady state.
MIN_WARM_S = 0.1


def _time_calls(fn, n_sets, steps, warmup, min_warm_s=0.0):
    """Average time per call (ms) over `steps` calls, HIP events on the launch stream, after
    at least `warmup` calls and min_warm_s seconds of calls (each input set at least once
    when min_warm_s > 0).  The counts go to call_counts()."""
    import torch
    n_w = 0
    while n_w < warmup:
        fn(n_w % n_sets)
        n_w += 1
    if min_warm_s > 0:
        # counted from here: a first call's one-time set-up (a library's kernel load) is not warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while n_w < n_sets or time.perf_counter() - t0 < min_warm_s:
            for _ in range(n_sets):
                fn(n_w % n_sets)
                n_w += 1
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i % n_sets)
    t1.record(stream)
    torch.cuda.synchronize()
    _COUNTS.update(warmup_calls=n_w, timed_calls=steps)
    return t0.elapsed_time(t1) / steps


_COUNTS = {}


def call_counts():
    """Warm-up and timed call counts of the last _time_calls."""
    return dict(_COUNTS)


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


def _timed(fn, n_sets, steps, warmup, stat_calls=None, min_warm_s=MIN_WARM_S):
    """(ms per call over the timed region, per-call statistics with the call counts: warm-up
    calls, then timed calls, then the statistics calls, in that order on the stream)."""
    ms = _time_calls(fn, n_sets, steps, warmup, min_warm_s)
    counts = call_counts()
    stats = _call_stats(fn, n_sets, stat_calls if stat_calls else max(10, min(steps, 100)))
    stats.update(counts)
    return ms, stats


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic__all_legs.txt")
CSRC = os.path.join(ROOT, "attention_shared_base_amd", "csrc")


def kernel_sources_sha():
    """sha256 (16 hex digits) over every kernel source of the library."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(leg):
    """HBM bytes per launch of a leg's dominant kernel from the committed counter
    summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain-copy calibration),
    with its source; (None, reason) when the kernel sources changed since."""
    try:
        rows, sha = {}, None
        for line in open(TRAFFIC_FILE):
            line = line.strip()
            if line.startswith("source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("leg "):
                f = dict(kv.split("=", 1) for kv in line.split()[2:])
                rows[line.split()[1]] = f
        if sha != kernel_sources_sha():
            return None, "counters were taken on other kernel sources"
        if leg not in rows:
            return None, "no counter record for this leg"
        return int(rows[leg]["traffic_bytes_per_launch"]), \
            f"profiles/{os.path.basename(TRAFFIC_FILE)} (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE; " \
            f"kernel {rows[leg]['kernel']})"
    except (OSError, KeyError, ValueError) as e:
        return None, f"no counter summary ({type(e).__name__})"


_FLOORS = {}


def read_floor(nbytes, calls=60):
    """The fastest plain read of nbytes this device gives (lra_ceiling_hbm_read): best of
    non-temporal / cached loads, grid-stride / chunked layouts and three grid sizes,
    rotated over buffers of >= 1 GiB in all so that the 256 MB Infinity Cache cannot
    serve repeats.  Measured once per size."""
    nbytes = -(-int(nbytes) // 16) * 16
    if nbytes in _FLOORS:
        return _FLOORS[nbytes]
    import torch
    import attention_shared_base_amd as lra
    n_sets = max(2, -(-(1 << 30) // nbytes))
    bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device="cuda") for i in range(n_sets)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for nt in (True, False):
        for chunked in (False, True):
            for n_wg in (2048, 4096, 8192):
                ms = _time_calls(lambda i: lra.ceiling_hbm_read(bufs[i], sink, n_workgroups=n_wg, nontemporal=nt,
                                                                chunked=chunked), n_sets, calls, 5, MIN_WARM_S / 2)
                if best is None or ms < best[0]:
                    best = (ms, nt, chunked, n_wg)
    ms, nt, chunked, n_wg = best
    dev_kernel = f"hbm_read{'_chunked' if chunked else ''}_kernel<{'true' if nt else 'false'}>"
    _FLOORS[nbytes] = {"bytes": nbytes, "us_per_call": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                       "kernel": f"lra_ceiling_hbm_read ({dev_kernel})", "device_kernel": dev_kernel,
                       "loads": "non-temporal" if nt else "cached",
                       "layout": "chunked" if chunked else "grid-stride", "workgroups": n_wg,
                       "buffers_rotated": n_sets, "calls": calls}
    del bufs
    return _FLOORS[nbytes]


def _roofline(leg, bound, achieved, floor_bytes=None):
    """The roofline object of a leg; for HBM-bound legs given floor_bytes, also the
    leg's rate as a fraction of a plain read of that many bytes on this device."""
    peak = HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS
    rl = {"bound": bound, "achieved": achieved, "peak": peak,
          "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "frac": achieved / peak}
    traffic, src = measured_traffic(leg)
    rl["traffic"] = traffic
    rl["traffic_source"] = src
    if floor_bytes:
        fl = read_floor(floor_bytes)
        rl["measured_read"] = fl
        rl["frac_of_measured_read"] = achieved / fl["gbs"]
    return rl


# ----------------------------------------------------------------------------- oracle timing

def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


@contextlib.contextmanager
def _one_core():
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            yield
    except ImportError:  # pragma: no cover
        yield


def _oracle_run(fn, min_seconds):
    """Run fn at least once and until min_seconds have passed: (first result, calls, seconds)."""
    t0 = time.perf_counter()
    res = fn()
    reps = 1
    while time.perf_counter() - t0 < min_seconds:
        fn()
        reps += 1
    return res, reps, time.perf_counter() - t0


def _cpu(value, unit, sample, threads=None):
    return {"value": value, "unit": unit, "cores": int(threads if threads else _blas_threads()),
            "kind": "oracle", "sample": sample, "host_cores": _host_cores()}


def _parity(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    max_abs = float(np.max(np.abs(err)))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    ok = bool(np.all(np.isfinite(got))) and (
        max_abs <= F32_MAX_ABS if dtype == "f32" else (max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2))
    return {"checked": what, "max_abs": max_abs, "rel_l2": rel,
            "bar": "max-abs 1e-5" if dtype == "f32" else "max-abs 2e-2 and rel-L2 1e-2", "pass": ok}


# ----------------------------------------------------------------------------- decode legs

class DecodeSet:
    """A seeded decode case uploaded in the kernel's page layouts."""

    def __init__(self, case, per_agent_lr=None):
        import workloads as w
        k, v, lk, lv = w.decode_device_layout(case.k_pool, case.v_pool, case.lk_pool, case.lv_pool)
        self.case = case
        self.q, self.k, self.v = map(_dev, (case.q, k, v))
        if per_agent_lr is None:
            self.lk, self.lv = _dev(lk), _dev(lv)
        else:  # [n_agents, n_pages, page, r] logical pools, one per agent
            lk_pa, lv_pa = per_agent_lr
            self.lk = _dev(lk_pa)
            self.lv = _dev(np.ascontiguousarray(lv_pa.transpose(0, 1, 3, 2)))
        self.crs = _dev(case.ctx_req_start())
        self.agent = _dev(case.req_agent)
        self.bt = _dev(case.block_table)
        self.clen = _dev(case.ctx_len)
        self.b_k, self.b_v = _dev(case.b_k), _dev(case.b_v)
        self.out = None


def _oracle_decode(case, rope_theta=None, requests=None, per_agent_lr=None):
    import oracle
    import workloads as w
    rope = None
    if rope_theta is not None:
        rope = oracle.rope_tables(max(int(case.ctx_len.max()), 1), case.d, rope_theta)
    lk, lv = (case.lk_pool, case.lv_pool) if per_agent_lr is None else per_agent_lr
    return oracle.decode_paged(w.widen(case.q), case.req_ctx, case.req_agent, w.widen(case.k_pool),
                               w.widen(case.v_pool), w.widen(lk), w.widen(lv), case.block_table,
                               case.ctx_len, w.widen(case.b_k), w.widen(case.b_v), rope=rope,
                               requests=requests)


def _decode_cases(n_sets, rank=16):
    import workloads as w
    if rank == 16:
        return [w.config2(layer=i) for i in range(n_sets)]
    # the same shapes and draws at another rank
    return [w.make_decode(2, dtype="bf16", ctx_lens=[8192] * 4, reqs=[(b // 4, b % 4) for b in range(16)],
                          n_agents=4, h_q=32, h_kv=8, d=128, r=rank, shuffle=False, layer=i)
            for i in range(n_sets)]


def _per_agent_lr(case, layer):
    """One seeded LR pool per agent, [n_agents, n_pages, page, r] (logical layout)."""
    import workloads as w
    from workloads.synth import TAG_LK, TAG_LV
    shape = (case.n_agents,) + tuple(case.lk_pool.shape)
    return (w.draw(102, TAG_LK, shape, 1.0, "bf16", layer), w.draw(102, TAG_LV, shape, 1.0, "bf16", layer))


def run_decode(steps, warmup, n_sets, rope_theta=None, per_agent=False, rank=16, min_warm_s=MIN_WARM_S):
    """Time lra_attn_decode over n_sets rotated seeded sets of the primary workload's shapes.
    Returns (case of set 0, ms per call, per-call stats, algorithmic bytes, set 0's output,
    set 0's per-agent LR pools or None)."""
    import torch
    import attention_shared_base_amd as lra
    cases = _decode_cases(n_sets, rank)
    pa = [_per_agent_lr(c, i) for i, c in enumerate(cases)] if per_agent else [None] * n_sets
    sets = [DecodeSet(c, p) for c, p in zip(cases, pa)]
    c0 = cases[0]
    mrpc = int(np.bincount(c0.req_ctx).max())
    max_len = int(c0.ctx_len.max())
    ws = torch.zeros(max(16, lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=rank, dtype=1, n_req=c0.n_req,
        n_ctx=c0.n_ctx, max_req_per_ctx=mrpc, max_ctx_len=max_len,
        lr_agent_stride=1 if per_agent else 0)), dtype=torch.uint8, device="cuda")
    for s in sets:
        s.out = torch.empty_like(s.q)
    cos = sin = None
    if rope_theta is not None:
        cos, sin = lra.rope_table(rope_theta, 128, max_len)

    # arguments checked and marshalled once per set (lra.prepare_decode): a timed call is
    # the C-ABI launch itself, as in a serving loop over fixed buffers
    prepared = [lra.prepare_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                                   max_req_per_ctx=mrpc, max_ctx_len=max_len, rope_cos=cos, rope_sin=sin,
                                   out=s.out, workspace=ws) for s in sets]

    def call(i):
        prepared[i]()

    ms, stats = _timed(call, n_sets, steps, warmup, max(20, min(steps, 200)), min_warm_s)
    nbytes = decode_bytes(c0.ctx_len, c0.n_req, len(np.unique(c0.req_agent)), 32, 8, 128, rank)
    if rope_theta is not None:
        nbytes += 2 * max_len * 64 * 4  # the cos / sin rows, read once
    if per_agent:  # every agent of a context reads its own L_k, L_v rows
        n_ag_ctx = len(np.unique(c0.req_agent[c0.req_ctx == 0]))
        nbytes += int(c0.ctx_len.sum()) * 2 * rank * 2 * (n_ag_ctx - 1)
    return c0, ms, stats, nbytes, _host(sets[0].out), pa[0]


def _decode_leg(name, workload, case, ms, stats, nbytes, got, oracle_fn, oracle_min_s, **extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    leg = {"workload": workload, "value": case.n_req / (ms * 1e-3), "unit": "tokens/s",
           "ms_per_call": ms, "call_us": stats,
           "roofline": _roofline(name, "hbm", gbs, nbytes),
           "algorithmic_bytes": nbytes}
    leg.update(UNCHECKED)
    if CHECK:
        ref, reps, el = _oracle_run(oracle_fn, oracle_min_s)
        leg["cpu_baseline"] = _cpu(reps * case.n_req / el, "tokens/s",
                                   f"full call (all {case.n_req} requests) on the timed set 0, "
                                   f"{reps}x in {el:.1f} s, float64 NumPy")
        leg["parity"] = _parity(got, ref, "bf16", f"set 0, all {case.n_req} requests")
        del leg["note_oracle"]
    leg.update(extra)
    return leg


def leg_decode_rope(steps, warmup, base_ms):
    """The primary decode workload with RoPE (theta 5e5) on the adapter key term: each
    request's key adapter is rebuilt at head dimension and rotated per page."""
    case, ms, stats, nbytes, got, _ = run_decode(steps, warmup, 4, rope_theta=500000.0)
    return _decode_leg(
        "decode_rope", "decode with RoPE on the adapter key: 16 requests over 4 shared 8192-token "
        "contexts, Hq32 Hkv8 d128 r16, theta 5e5, bf16", case, ms, stats, nbytes, got,
        lambda: _oracle_decode(case, rope_theta=500000.0), 3.0, time_vs_no_rope=ms / base_ms if base_ms else None)


def leg_decode_qkvo_r4(steps, warmup):
    """The pages' query/key/value/output LoRA setting (LRAgent App. D.1): rank 4 with RoPE on
    the adapter key, against the plain rank-4 call on the same shapes."""
    _, ms_plain, _, _, _, _ = run_decode(steps, warmup, 4, rank=4)
    case, ms, stats, nbytes, got, _ = run_decode(steps, warmup, 4, rope_theta=500000.0, rank=4)
    return _decode_leg(
        "decode_qkvo_r4", "decode, rank-4 LoRA with RoPE on the adapter key (qkvo setting): 16 "
        "requests over 4 shared 8192-token contexts, Hq32 Hkv8 d128 r4, theta 5e5, bf16",
        case, ms, stats, nbytes, got, lambda: _oracle_decode(case, rope_theta=500000.0), 3.0,
        ms_per_call_without_rope=ms_plain, time_vs_no_rope=ms / ms_plain)


def leg_decode_per_agent(steps, warmup, base_ms):
    """The primary decode workload with one LR cache per agent (BaseShared / PreLRShared with
    per-agent A): each request reads its agent's L_k, L_v pages beside the shared base pages."""
    case, ms, stats, nbytes, got, pa = run_decode(steps, warmup, 4, per_agent=True)
    return _decode_leg(
        "decode_per_agent", "decode with one LR cache per agent: 16 requests over 4 shared "
        "8192-token contexts (4 agents each), Hq32 Hkv8 d128 r16, bf16", case, ms, stats, nbytes,
        got, lambda: _oracle_decode(case, per_agent_lr=pa), 3.0, time_vs_shared_lr=ms / base_ms if base_ms else None)


def leg_naive_decode(steps, warmup, base_ms, primary_cpu):
    """Baseline of the Flash-LoRA comparison on the primary decode workload: every
    request's K, V materialised at head dimension (expansion kernel), then plain decode
    attention over the per-request caches.  Reported next to the method's time."""
    import workloads as w
    import attention_shared_base_amd as lra
    n_sets = 2
    cases = [w.config2(layer=i) for i in range(n_sets)]
    sets = [DecodeSet(c) for c in cases]
    c0 = cases[0]
    mrpc = int(np.bincount(c0.req_ctx).max())
    max_len = int(c0.ctx_len.max())
    scratch = [{} for _ in sets]
    outs = [None] * n_sets

    def call(i):
        s = sets[i]
        outs[i] = lra.naive_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k,
                                   s.b_v, max_req_per_ctx=mrpc, max_ctx_len=max_len,
                                   scratch=scratch[i])

    ms, stats = _timed(call, n_sets, steps, warmup, 10)
    n_tok = int(c0.ctx_len[c0.req_ctx].sum())
    # bytes the baseline moves: base K, V read and the expanded K, V written per request,
    # the expanded K, V read again by the attention (per KV head, bf16)
    nbytes = 3 * n_tok * 8 * 128 * 2 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    req = [0, 5, 10, 15]
    leg = {
        "workload": "baseline without Flash-LoRA-Attention: primary decode workload with each "
                    "request's K = K_base + L_k B_k, V = V_base + L_v B_v written to HBM, then "
                    "plain decode attention over the per-request caches",
        "value": c0.n_req / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "call_us": stats,
        "method_speedup": ms / base_ms if base_ms else None,
        "roofline": _roofline("naive_decode", "hbm", gbs), "algorithmic_bytes": nbytes,
        "cpu_baseline": dict(primary_cpu, sample="the primary leg's oracle timing (the same "
                                                 "workload; the oracle materialises in either case)"),
        "parity": None,
    }
    if CHECK:
        ref = _oracle_decode(c0, requests=req)
        leg["parity"] = _parity(_host(outs[0])[req], ref[req], "bf16", f"set 0, requests {req}")
    return leg


def leg_agent_scaling(steps, warmup, primary_cpu):
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

        ms = _time_calls(call, len(sets), steps, warmup, MIN_WARM_S)
        ms_naive = _time_calls(call_naive, len(sets), max(4, steps // 20), 2, MIN_WARM_S)
        table[str(rpc)] = {"decode_us": ms * 1e3, "naive_us": ms_naive * 1e3,
                           "decode_tokens_per_s": n_req / (ms * 1e-3)}
        del scratch, ws
        torch.cuda.empty_cache()
    t1, t4, t16 = (table[k]["decode_us"] for k in ("1", "4", "16"))
    return {"workload": "decode over 4 shared 8192-token contexts, Hq32 Hkv8 d128 r16, with 1, 2, 4, "
                        "8, 16 requests (agents) per context; method and naive materialising baseline",
            "value": t4 / t1, "unit": "x (time at 4 agents per context / time at 1)",
            "time_16_vs_1": t16 / t1, "per_agents": table, "roofline": None,
            "cpu_baseline": dict(primary_cpu, sample="the primary leg's oracle timing: the oracle's "
                                                     "cost is per request, whatever the sharing"),
            "parity": None,
            "note": "scaling study (ratio, no roofline): sharing the base and LR caches across agents; "
                    "its kernels are the primary leg's, checked there and in the tests"}


def leg_paged_decode(steps, warmup):
    """Seeded paged decode: 32 contexts of U[4096, 65536] tokens, shuffled 16-token pages,
    32 requests over 8 agents, r 32 (about 5.4 GB of caches, beyond the Infinity Cache)."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    t0 = time.perf_counter()
    case = w.config4()
    s = DecodeSet(case)
    _log(f"paged_decode: seeded inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    lens = case.ctx_len
    max_len = int(lens.max())
    s.out = torch.empty_like(s.q)
    ws = torch.zeros(lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=32, dtype=1, n_req=32, n_ctx=32,
        max_req_per_ctx=1, max_ctx_len=max_len), dtype=torch.uint8, device="cuda")

    prepared = lra.prepare_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                                  max_req_per_ctx=1, max_ctx_len=max_len, out=s.out, workspace=ws)

    def call(_):
        prepared()

    ms, stats = _timed(call, 1, steps, warmup, 10)
    del prepared
    nbytes = decode_bytes(lens, 32, 8, 32, 8, 128, 32)
    gbs = nbytes / (ms * 1e-3) / 1e9
    got = _host(s.out)
    # oracle on a sample of requests (shortest, longest and two more), timed and scaled to the
    # whole call by context tokens (the oracle's work is linear in them)
    sample = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 5, 18})
    del s
    torch.cuda.empty_cache()
    leg = {"workload": "paged decode: 32 contexts of U[4096,65536] tokens (sum %d), shuffled "
                        "16-token pages, 32 requests over 8 agents, Hq32 Hkv8 d128 r32, bf16"
                        % int(lens.sum()),
            "value": 32 / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "call_us": stats,
            "roofline": _roofline("paged_decode", "hbm", gbs, nbytes), "algorithmic_bytes": nbytes,
            "data": "seeded host generator (workload 4 of the tests)"}
    leg.update(UNCHECKED)
    if CHECK:
        sub = w.decode_subset(case, sample)  # only the sampled contexts' pages (data movement)
        ref, reps, el = _oracle_run(lambda: _oracle_decode(sub), 0.0)
        tok_sample = int(lens[sample].sum())
        t_call = el / reps * int(lens.sum()) / tok_sample
        leg["cpu_baseline"] = _cpu(32 / t_call, "tokens/s",
                                   f"requests {sample} ({tok_sample} of {int(lens.sum())} context "
                                   f"tokens) in {el / reps:.1f} s, scaled to the whole call by tokens")
        leg["parity"] = _parity(got[sample], ref, "bf16", f"requests {sample}")
        del leg["note_oracle"]
    return leg


def leg_workload1_fp32(steps, warmup):
    """The fp32 parity workload (2 agents over one 256-token context, Hq4 Hkv2 d64 r8): call time
    of its decode (2 requests) and its causal prefill (2 x 16 new tokens).  Launch-latency bound
    (a 278 KB working set); reported as time only."""
    import torch
    import attention_shared_base_amd as lra
    import oracle
    import workloads as w
    dec, pre = w.config1()
    s = DecodeSet(dec)
    d_out = torch.empty_like(s.q)
    q, agent = _dev(pre.q), _dev(pre.req_agent)
    k, v, lk, lv, bk, bv = map(_dev, (pre.k_base, pre.v_base, pre.l_k, pre.l_v, pre.b_k, pre.b_v))
    p_out = torch.empty_like(q)

    # arguments checked and marshalled once: the timed calls are the C-ABI launches
    prep_d = lra.prepare_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k, s.b_v,
                                max_req_per_ctx=2, max_ctx_len=256, out=d_out)
    prep_p = lra.prepare_prefill(q, agent, k, v, lk, lv, bk, bv, out=p_out)

    def call_d(_):
        prep_d()

    def call_p(_):
        prep_p()

    ms_d, stats_d = _timed(call_d, 1, steps, warmup)
    ms_p, stats_p = _timed(call_p, 1, steps, warmup)
    o_dec = lambda: _oracle_decode(dec)  # noqa: E731
    o_pre = lambda: oracle.prefill(w.widen(pre.q), pre.req_agent, w.widen(pre.k_base),  # noqa: E731
                                   w.widen(pre.v_base), w.widen(pre.l_k), w.widen(pre.l_v),
                                   w.widen(pre.b_k), w.widen(pre.b_v))
    leg = {"workload": "fp32 parity workload: 2 agents over one 256-token context (240 + 16 new), "
                        "Hq4 Hkv2 d64 r8; decode of 2 requests and prefill of 2 x 16 tokens",
            "value": ms_d * 1e3, "unit": "us per decode call", "higher_is_better": False,
            "ms_per_call": ms_d, "call_us": stats_d,
            "prefill_us_per_call": ms_p * 1e3, "prefill_call_us": stats_p,
            "roofline": None,
            "note": "launch-latency bound (278 KB working set): time only, no roofline"}
    leg.update(UNCHECKED)
    if CHECK:
        ref_d, rd, ed = _oracle_run(o_dec, 2.0)
        ref_p, rp, ep = _oracle_run(o_pre, 2.0)
        with _one_core():
            _, rd1, ed1 = _oracle_run(o_dec, 1.0)
            _, rp1, ep1 = _oracle_run(o_pre, 1.0)
        leg["cpu_baseline"] = _cpu(ed / rd * 1e6, "us per decode call",
                                   f"full decode call repeated {rd}x in {ed:.1f} s; prefill "
                                   f"{ep / rp * 1e6:.0f} us per call")
        leg["cpu_baseline_1core"] = _cpu(ed1 / rd1 * 1e6, "us per decode call",
                                         f"one BLAS thread: decode {rd1}x in {ed1:.1f} s; prefill "
                                         f"{ep1 / rp1 * 1e6:.0f} us per call", threads=1)
        leg["parity"] = {"decode": _parity(_host(d_out), ref_d, "f32", "both requests"),
                         "prefill": _parity(_host(p_out), ref_p, "f32", "all 2 x 16 rows")}
        del leg["note_oracle"]
    return leg


# ----------------------------------------------------------------------------- prefill legs

def _oracle_prefill(case, rows=None, requests=None, l_k=None, l_v=None):
    import oracle
    import workloads as w
    rope = (oracle.rope_tables(case.kv_len, case.d, case.rope_theta)
            if case.rope_theta is not None else None)
    q = w.widen(case.q)
    agents = case.req_agent
    if requests is not None:
        q, agents = q[requests], agents[requests]
    return oracle.prefill(q, agents, w.widen(case.k_base), w.widen(case.v_base),
                          w.widen(case.l_k) if l_k is None else l_k,
                          w.widen(case.l_v) if l_v is None else l_v,
                          w.widen(case.b_k), w.widen(case.b_v), rope=rope, rows=rows)


def leg_prefill_rope(steps, warmup, n_sets=6):
    """Seeded workload 3: 512 new tokens over a 16384-token shared context, 4 agents, RoPE 5e5
    on the adapter key; n_sets independent sets of about 86 MB rotated."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    cases = [w.config3(layer=i) for i in range(n_sets)]
    sets = []
    for c in cases:
        sets.append(dict(q=_dev(c.q), k=_dev(c.k_base), v=_dev(c.v_base), lk=_dev(c.l_k),
                         lv=_dev(c.l_v), bk=_dev(c.b_k), bv=_dev(c.b_v)))
        sets[-1]["out"] = torch.empty_like(sets[-1]["q"])
    c0 = cases[0]
    agent = _dev(c0.req_agent)
    cos, sin = lra.rope_table(500000.0, 128, c0.kv_len)

    prepared = [lra.prepare_prefill(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bk"], s["bv"],
                                    rope_cos=cos, rope_sin=sin, out=s["out"]) for s in sets]

    def call(i):
        prepared[i]()

    ms, stats = _timed(call, n_sets, steps, warmup, 20)
    got = _host(sets[0]["out"])
    fl = prefill_flops(4, 512, c0.kv_len, 32, 8, 128, 16, rope=True)
    tf = fl / (ms * 1e-3) / 1e12
    set_mb = sum(t.numel() * t.element_size() for t in sets[0].values()) / 1e6
    leg = {"workload": "chunked prefill: 512 new tokens over 16384 shared, 4 agents, RoPE "
                        "theta 5e5 on the adapter key term, Hq32 Hkv8 d128 r16, bf16",
            "value": tf, "unit": "TFLOP/s", "ms_per_call": ms, "call_us": stats,
            "roofline": _roofline("prefill_rope", "mfma", tf), "algorithmic_flops": fl,
            "input_sets_rotated": n_sets, "input_set_mb": set_mb,
            "data": "seeded host generator (workload 3 of the tests), one draw per set"}
    leg.update(UNCHECKED)
    if CHECK:
        ref, reps, el = _oracle_run(lambda: _oracle_prefill(c0), 0.0)
        leg["cpu_baseline"] = _cpu(fl / el * reps / 1e12, "TFLOP/s",
                                   f"full call (4 requests x 512 rows) on set 0 in {el:.1f} s")
        leg["parity"] = _parity(got, ref, "bf16", "set 0, all 4 x 512 x 32 rows")
        del leg["note_oracle"]
    return leg


def leg_prefill_paged(steps, warmup, base_ms, n_sets=6):
    """Workload 3 with the context in shuffled 16-token pages (lra_attn_prefill_paged)."""
    import torch
    import attention_shared_base_amd as lra
    import oracle
    import workloads as w
    cases = [w.config3(layer=i) for i in range(n_sets)]
    c0 = cases[0]
    kv_len = c0.kv_len
    n_pages = (kv_len + 15) // 16
    sets = []
    for i, c in enumerate(cases):
        ids = w.rng_for(300 + i, 12).permutation(n_pages)
        kp, lkp = w.paginate(c.k_base, c.l_k, ids, n_pages, 16)
        vp, lvp = w.paginate(c.v_base, c.l_v, ids, n_pages, 16)
        k, v, lk, lv = w.decode_device_layout(kp, vp, lkp, lvp)
        sets.append(dict(q=_dev(c.q), k=_dev(k), v=_dev(v), lk=_dev(lk), lv=_dev(lv),
                         bk=_dev(c.b_k), bv=_dev(c.b_v), bt=_dev(ids.astype(np.int32))))
        sets[-1]["out"] = torch.empty_like(sets[-1]["q"])
        if i == 0:
            pools0 = (kp, vp, lkp, lvp, ids)
    agent = _dev(c0.req_agent)
    cos, sin = lra.rope_table(500000.0, 128, kv_len)

    def call(i):  # the pages are read in place
        s = sets[i]
        lra.prefill_paged(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bt"], kv_len,
                          s["bk"], s["bv"], rope_cos=cos, rope_sin=sin, out=s["out"])

    ms, stats = _timed(call, n_sets, steps, warmup, 20)
    got = _host(sets[0]["out"])
    # the staged path (gather into a contiguous workspace, then the contiguous prefill)
    ws = torch.empty(lra.prefill_paged_staged_workspace_size(n_q_heads=32, n_kv_heads=8, head_dim=128,
                                                             rank=16, kv_len=kv_len) + 16,
                     dtype=torch.uint8, device="cuda")

    def call_staged(i):
        s = sets[i]
        lra.prefill_paged_staged(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bt"], kv_len,
                                 s["bk"], s["bv"], rope_cos=cos, rope_sin=sin, out=s["out"], workspace=ws)

    # (half the timed calls: the direct path stays the leg's dominant kernel in a profile)
    ms_staged, _ = _timed(call_staged, n_sets, max(steps // 2, 10), warmup, 10)
    # every set was called again by the staged path: set 0's output is its own
    staged_equal = bool(np.array_equal(_host(sets[0]["out"]), got))
    del ws
    fl = prefill_flops(4, 512, kv_len, 32, 8, 128, 16, rope=True)
    tf = fl / (ms * 1e-3) / 1e12
    kp, vp, lkp, lvp, ids = pools0

    def oracle_paged():  # the oracle gathers the pages itself, then prefills (request 0)
        kb, lk = oracle.gather_pages(w.widen(kp), w.widen(lkp), ids, kv_len)
        vb, lv = oracle.gather_pages(w.widen(vp), w.widen(lvp), ids, kv_len)
        return oracle.prefill(w.widen(c0.q[:1]), c0.req_agent[:1], kb, vb, lk, lv, w.widen(c0.b_k),
                              w.widen(c0.b_v), rope=oracle.rope_tables(kv_len, 128, 500000.0))

    leg = {"workload": "paged chunked prefill: the prefill leg's workload (512 new tokens over "
                        "16384, 4 agents, RoPE) with the context in shuffled 16-token pages",
            "value": tf, "unit": "TFLOP/s", "ms_per_call": ms, "call_us": stats,
            "time_vs_contiguous": ms / base_ms if base_ms else None,
            "staged": {"ms_per_call": ms_staged, "time_vs_direct": ms_staged / ms,
                       "output_equal_to_direct": staged_equal,
                       "workspace_mb": round(lra.prefill_paged_staged_workspace_size(
                           n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, kv_len=kv_len) / 1e6, 1)},
            "roofline": _roofline("prefill_paged", "mfma", tf), "algorithmic_flops": fl,
            "input_sets_rotated": n_sets,
            "data": "seeded host generator (workload 3), shuffled pages per set"}
    leg.update(UNCHECKED)
    if CHECK:
        ref, reps, el = _oracle_run(oracle_paged, 0.0)
        leg["cpu_baseline"] = _cpu(fl / 4 / (el / reps) / 1e12, "TFLOP/s",
                                   f"request 0 of 4 (page gather + 512 rows) on set 0 in "
                                   f"{el / reps:.1f} s; rate of a quarter of the call's flops")
        leg["parity"] = _parity(got[:1], ref, "bf16", "set 0, request 0 (512 x 32 rows)")
        del leg["note_oracle"]
    return leg


def leg_naive_prefill(steps, warmup, base_ms, n_sets=6):
    """Baseline of the Flash-LoRA comparison on workload 3 (512 new tokens over 16384, 4
    agents, RoPE): each request's K_base + rot(L_k B_k) and V_base + L_v B_v written to HBM
    (lra_naive_prefill), then plain causal attention over the per-request caches."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    cases = [w.config3(layer=i) for i in range(n_sets)]
    sets = []
    for c in cases:
        sets.append(dict(q=_dev(c.q), k=_dev(c.k_base), v=_dev(c.v_base), lk=_dev(c.l_k),
                         lv=_dev(c.l_v), bk=_dev(c.b_k), bv=_dev(c.b_v)))
        sets[-1]["out"] = torch.empty_like(sets[-1]["q"])
    c0 = cases[0]
    agent = _dev(c0.req_agent)
    cos, sin = lra.rope_table(500000.0, 128, c0.kv_len)
    ws = torch.empty(lra.naive_prefill_workspace_size(n_q_heads=32, n_kv_heads=8, head_dim=128,
                                                      rank=16, n_req=4, kv_len=c0.kv_len),
                     dtype=torch.uint8, device="cuda")

    def call(i):
        s = sets[i]
        lra.naive_prefill(s["q"], agent, s["k"], s["v"], s["lk"], s["lv"], s["bk"], s["bv"],
                          rope_cos=cos, rope_sin=sin, out=s["out"], workspace=ws)

    ms, stats = _timed(call, n_sets, steps, warmup, 20)
    fl = prefill_flops(4, 512, c0.kv_len, 32, 8, 128, 16, rope=True)
    tf = fl / (ms * 1e-3) / 1e12
    leg = {"workload": "baseline without Flash-LoRA-Attention: workload 3 (512 new tokens over "
                       "16384, 4 agents, RoPE) with each request's K = K_base + rot(L_k B_k), "
                       "V = V_base + L_v B_v written to HBM, then plain causal attention",
           "value": tf, "unit": "TFLOP/s (the method's algorithmic flops / baseline time)",
           "ms_per_call": ms, "call_us": stats,
           "method_speedup": ms / base_ms if base_ms else None,
           "roofline": _roofline("naive_prefill", "mfma", tf), "algorithmic_flops": fl,
           "input_sets_rotated": n_sets}
    leg.update(UNCHECKED)
    if CHECK:
        rows = np.unique(np.linspace(0, 511, 16).astype(np.int64))
        ref, reps, el = _oracle_run(lambda: _oracle_prefill(c0, rows=rows), 0.0)
        leg["cpu_baseline"] = _cpu(fl * len(rows) / 512 / (el / reps) / 1e12, "TFLOP/s",
                                   f"16 of 512 rows of all 4 requests on set 0 in {el / reps:.1f} s, "
                                   f"scaled by rows (the oracle materialises either way)")
        leg["parity"] = _parity(_host(sets[0]["out"])[:, rows], ref, "bf16",
                                "set 0, 16 rows (first and last included) x 4 requests x 32 heads")
        del leg["note_oracle"]
    return leg


def leg_naive_paged_decode(steps, warmup, base_ms):
    """Baseline of the Flash-LoRA comparison on workload 4 (32 shuffled contexts of 4k-64k
    tokens, r 32): each request's K, V expanded to pages of its own, then plain decode."""
    import torch
    import attention_shared_base_amd as lra
    import workloads as w
    case = w.config4()
    s = DecodeSet(case)
    lens = case.ctx_len
    max_len = int(lens.max())
    scratch = {}
    outs = [None]

    def call(_):
        outs[0] = lra.naive_decode(s.q, s.crs, s.agent, s.k, s.v, s.lk, s.lv, s.bt, s.clen, s.b_k,
                                   s.b_v, max_req_per_ctx=1, max_ctx_len=max_len, scratch=scratch)

    ms, stats = _timed(call, 1, steps, warmup, 5)
    n_tok = int(lens.sum())
    nbytes = 3 * n_tok * 8 * 128 * 2 * 2  # base read, expanded written, expanded read
    gbs = nbytes / (ms * 1e-3) / 1e9
    got = _host(outs[0])
    leg = {"workload": "baseline without Flash-LoRA-Attention: workload 4 (32 contexts of "
                       "U[4096,65536] tokens, shuffled pages, r 32) with each request's K, V "
                       "materialised to pages of its own, then plain decode",
           "value": 32 / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "call_us": stats,
           "method_speedup": ms / base_ms if base_ms else None,
           "roofline": _roofline("naive_paged_decode", "hbm", gbs), "algorithmic_bytes": nbytes}
    leg.update(UNCHECKED)
    del s, scratch
    torch.cuda.empty_cache()
    if CHECK:
        sample = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7, 22})
        sub = w.decode_subset(case, sample)
        ref, reps, el = _oracle_run(lambda: _oracle_decode(sub), 0.0)
        t_call = el / reps * n_tok / int(lens[sample].sum())
        leg["cpu_baseline"] = _cpu(32 / t_call, "tokens/s",
                                   f"requests {sample} in {el / reps:.1f} s, scaled by context tokens")
        leg["parity"] = _parity(got[sample], ref, "bf16", f"requests {sample}")
        del leg["note_oracle"]
    return leg


def leg_lr_build(steps, warmup, n_sets=8):
    """Seeded LR-cache build of one 4096-token layer: L = X [A_k | A_v], r 16."""
    import torch
    import attention_shared_base_amd as lra
    import oracle
    import workloads as w
    n_tok, d_model, r = 4096, 4096, 16
    cases = [w.make_lr_build(5, dtype="bf16", n_tok=n_tok, d_model=d_model, r=r, layer=i)
             for i in range(n_sets)]
    sets = [dict(x=_dev(c.x), ak=_dev(c.a_k), av=_dev(c.a_v),
                 lk=torch.empty((n_tok, r), dtype=torch.bfloat16, device="cuda"),
                 lv=torch.empty((n_tok, r), dtype=torch.bfloat16, device="cuda")) for c in cases]
    # one zero-filled workspace for every call (the calls leave it ready)
    n_ws = lra.lr_cache_build_workspace_size(dtype=1, n_tok=n_tok, d_model=d_model, rank=r)
    ws = torch.zeros(max(n_ws, 16), dtype=torch.uint8, device="cuda")

    def call(i):
        s = sets[i]
        lra.lr_cache_build(s["x"], s["ak"], s["av"], s["lk"], s["lv"], workspace=ws)

    ms, stats = _timed(call, n_sets, steps, warmup)
    nbytes = lr_build_bytes(n_tok, d_model, r)
    gbs = nbytes / (ms * 1e-3) / 1e9
    c0 = cases[0]
    leg = {"workload": "LR-cache build L = X [A_k|A_v]: X [4096, 4096] bf16, r 16",
            "value": gbs, "unit": "GB/s", "ms_per_call": ms, "call_us": stats,
            "roofline": _roofline("lr_build", "hbm", gbs, nbytes), "algorithmic_bytes": nbytes,
            "input_sets_rotated": n_sets}
    leg.update(UNCHECKED)
    if CHECK:
        (rk, rv), reps, el = _oracle_run(
            lambda: oracle.lr_cache_build(w.widen(c0.x), w.widen(c0.a_k).T, w.widen(c0.a_v).T), 2.0)
        got = np.concatenate([_host(sets[0]["lk"]), _host(sets[0]["lv"])], axis=1)
        leg["cpu_baseline"] = _cpu(nbytes / (el / reps) / 1e9, "GB/s",
                                   f"X A in float64 on set 0, {reps}x in {el:.1f} s")
        leg["parity"] = _parity(got, np.concatenate([rk, rv], axis=1), "bf16",
                                "set 0, all 4096 x 32 outputs")
        del leg["note_oracle"]
    return leg


def leg_prelr_step(steps, warmup, n_layers=32):
    """PreLRShared step: per layer, LR build of 4096 new rows, then 8 agents' prefill.

    32 layers of LLaMA-3.1-8B attention shape, each with its own buffers: X
    [4096, 4096], A_k/A_v [16, 4096], K_base/V_base [8, 135168, 128] (131072
    old + 4096 new tokens), L_k/L_v [135168, 16] (old rows given, new rows built
    in the step), per-agent Q [4096, 32, 128] and B [16, 1024].  Inputs are
    drawn on the GPU (torch Philox, 27 GB) with the distributions of the seeded
    host generator; the last layer's outputs are checked against the oracle.
    """
    import torch
    import attention_shared_base_amd as lra
    import oracle
    n_new, n_old, d_model, h_q, h_kv, d, r, n_ag = 4096, 131072, 4096, 32, 8, 128, 16, 8
    kv_len = n_old + n_new
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    layers = []
    for _ in range(n_layers):
        layers.append(dict(
            x=_randn_bf16((n_new, d_model), 1.0, gen),
            ak=_randn_bf16((r, d_model), 1.0 / 64, gen), av=_randn_bf16((r, d_model), 1.0 / 64, gen),
            k=_randn_bf16((h_kv, kv_len, d), 1.0, gen), v=_randn_bf16((h_kv, kv_len, d), 1.0, gen),
            lk=_randn_bf16((kv_len, r), 1.0, gen), lv=_randn_bf16((kv_len, r), 1.0, gen),
            q=_randn_bf16((n_ag, n_new, h_q, d), 1.0, gen),
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

    ms, stats = _timed(call, 1, steps, warmup, 3)
    fl_layer_attn = prefill_flops(n_ag, n_new, kv_len, h_q, h_kv, d, r, rope=False)
    fl_layer_lr = 2 * n_new * d_model * 2 * r
    fl = n_layers * (fl_layer_attn + fl_layer_lr)
    tf = fl / (ms * 1e-3) / 1e12
    leg = {"workload": "PreLRShared step: 32 layers x (LR build X[4096,4096]·[A_k|A_v] r16, then "
                       "8 agents' prefill of 4096 new tokens over 131072 shared), Hq32 Hkv8 d128, bf16",
           "value": tf, "unit": "TFLOP/s", "ms_per_call": ms, "call_us": stats,
           "roofline": _roofline("prelr_step", "mfma", tf), "algorithmic_flops": fl,
           "data": "torch Philox draws on the GPU with the seeded generator's distributions"}
    leg.update(UNCHECKED)
    if not CHECK:
        return leg
    del leg["note_oracle"]
    # ---- oracle on the last layer (whose rows `out` holds): LR build vs X A in float64, and
    # attention of 16 sampled rows (first and last included) of all 8 agents, end to end (the
    # oracle's own X A rows as the new LR rows).  One (agent, layer) pair is timed at two row counts; the fit
    # t(n) = a + b n (a: materialising K and V, b: per row) gives the pair's full-call time,
    # extrapolated x 256 pairs plus 32 LR builds.
    L = layers[-1]
    got = _host(out)
    x, ak, av = _host(L["x"]), _host(L["ak"]), _host(L["av"])
    (rk, rv), reps_lr, el_lr = _oracle_run(lambda: oracle.lr_cache_build(x, ak.T, av.T), 0.0)
    lk, lv = _host(L["lk"]), _host(L["lv"])
    lr_par = _parity(np.concatenate([lk[n_old:], lv[n_old:]], 1), np.concatenate([rk, rv], 1),
                     "bf16", "last layer's 4096 new LR rows (both caches) vs X A in float64")
    lk_o, lv_o = np.concatenate([lk[:n_old], rk]), np.concatenate([lv[:n_old], rv])
    kb, vb = _host(L["k"]), _host(L["v"])
    bk, bv = _host(L["bk"]), _host(L["bv"])
    rows16 = np.unique(np.linspace(0, n_new - 1, 16).astype(np.int64))
    rows48 = np.unique(np.linspace(0, n_new - 1, 48).astype(np.int64))
    ok_max, ok_rel, ok = 0.0, 0.0, True
    t16 = t48 = None
    for a in range(n_ag):
        qa = _host(L["q"][a:a + 1])
        t0 = time.perf_counter()
        ref = oracle.prefill(qa, np.array([a]), kb, vb, lk_o, lv_o, bk, bv, rows=rows16)
        t = time.perf_counter() - t0
        if a == 0:
            t16 = t
            t0 = time.perf_counter()
            oracle.prefill(qa, np.array([a]), kb, vb, lk_o, lv_o, bk, bv, rows=rows48)
            t48 = time.perf_counter() - t0
        p = _parity(got[a:a + 1, rows16], ref, "bf16", "")
        ok_max, ok_rel, ok = max(ok_max, p["max_abs"]), max(ok_rel, p["rel_l2"]), ok and p["pass"]
    b_row = max((t48 - t16) / (len(rows48) - len(rows16)), 0.0)
    a_fix = max(t16 - b_row * len(rows16), 0.0)
    t_pair = a_fix + b_row * n_new
    t_total = n_layers * n_ag * t_pair + n_layers * el_lr / reps_lr
    leg.update({"cpu_baseline": _cpu(fl / t_total / 1e12, "TFLOP/s",
                                 f"extrapolated: one (agent, layer) pair timed at 16 and 48 query rows "
                                 f"({t16:.1f} s, {t48:.1f} s; fit {a_fix:.1f} s + {b_row * 1e3:.0f} ms "
                                 f"per row -> {t_pair:.0f} s per pair), x 256 pairs + 32 LR builds "
                                 f"({el_lr / reps_lr:.2f} s each) = {t_total / 3600:.1f} h per step"),
            "parity": {"attention": {"checked": "last layer, 16 rows (first and last included) of "
                                                "each of the 8 agents, end to end (new LR rows: the "
                                                "oracle's X A in float64)",
                                     "max_abs": ok_max, "rel_l2": ok_rel,
                                     "bar": "max-abs 2e-2 and rel-L2 1e-2", "pass": ok},
                       "lr_build": lr_par}})
    return leg


def leg_ceilings(steps, warmup):
    """What this device sustains, as reference points for the rooflines: the plain read
    stream at 1 GiB, the bf16 MFMA stream with both operands in registers and with the
    B operand read from LDS for every MFMA, and torch's bf16 GEMM (8192^3)."""
    import torch
    import attention_shared_base_amd as lra
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    rd = read_floor(1 << 30)
    n_wg, iters = 2048, 2048  # 8 workgroups (32 wavefronts) per CU, about a millisecond a call
    mfma = {}
    for lds, key in ((0, "register_operands"), (1, "lds_operand_b"), (2, "lds_operands_ab")):
        flops = n_wg * iters * 524288
        ms = _time_calls(lambda i: lra.ceiling_mfma_bf16(sink, n_workgroups=n_wg, iters=iters, lds_operands=lds),
                         1, max(10, steps // 10), 3, MIN_WARM_S)
        tf = flops / (ms * 1e-3) / 1e12
        mfma[key] = {
            "kernel": "lra_ceiling_mfma_bf16", "lds_operands": lds, "flops_per_call": flops, "ms_per_call": ms,
            "tflops": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS,
            # v_mfma_f32_32x32x16_bf16 at one issue per 8 passes on every SIMD, at the
            # published 2.4 GHz, is the published peak; this is the clock that would
            # give the measured rate if the MFMA pipes never idled
            "clock_ghz_if_pipes_never_idle": 2.4 * tf / BF16_PEAK_TFLOPS,
            # LDS operand bytes read per CU per second (1 KB per wavefront per operand per MFMA)
            "lds_gb_per_s_per_cu": lds * n_wg * 4 * iters * 4 * 1024 / (ms * 1e-3) / 256 / 1e9}
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn((8192, 8192), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty_like(a)
    gms = _time_calls(lambda i: torch.mm(a, b, out=c), 1, max(10, steps // 10), 3, MIN_WARM_S)
    gtf = 2 * 8192 ** 3 / (gms * 1e-3) / 1e12
    best = max(v["tflops"] for v in mfma.values())
    leg = {"workload": "device ceilings: HBM read stream of 1 GiB; bf16 MFMA stream, 2048 workgroups x "
                       "2048 rounds; torch bf16 GEMM 8192^3",
           "value": best, "unit": "TFLOP/s", "ms_per_call": mfma["register_operands"]["ms_per_call"],
           "roofline": _roofline("ceilings", "mfma", best),
           "hbm_read": dict(rd, frac_of_peak=rd["gbs"] / HBM_PEAK_GBS,
                            traffic=measured_traffic(f"ceilings_read_{rd['device_kernel']}")[0]),
           "mfma_bf16": mfma,
           "torch_gemm_bf16": {"shape": [8192, 8192, 8192], "ms_per_call": gms, "tflops": gtf,
                               "frac_of_peak": gtf / BF16_PEAK_TFLOPS},
           "cpu_baseline": None, "parity": None,
           "note_oracle": "device probes: nothing to compare with the oracle"}
    return leg


# ----------------------------------------------------------------------------- misc

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


def primary_cpu_baselines(case, got, min_seconds=6.0):
    """The float64 oracle on the primary workload's timed set 0: all BLAS threads, then one."""
    ref, reps, el = _oracle_run(lambda: _oracle_decode(case), min_seconds)
    cpu = _cpu(reps * case.n_req / el, "tokens/s",
               f"full decode call of the primary workload's set 0 (16 requests x 8192 keys), "
               f"repeated {reps}x in {el:.1f} s, float64 NumPy")
    with _one_core():
        _, r1, e1 = _oracle_run(lambda: _oracle_decode(case), 2.0)
    cpu1 = _cpu(r1 * case.n_req / e1, "tokens/s",
                f"the same call with one BLAS thread, repeated {r1}x in {e1:.1f} s", threads=1)
    return cpu, cpu1, _parity(got, ref, "bf16", "set 0, all 16 requests")


def _extra_legs(args, base_ms, primary_cpu, extra=None):
    """The extra legs by name (base_ms: the primary decode's time, for ratios)."""
    extra = {} if extra is None else extra
    pcpu = primary_cpu if primary_cpu else _cpu(None, "tokens/s", "primary leg not run")
    mid = max(10, args.steps)          # sub-millisecond to millisecond calls
    slow = max(5, args.steps // 4)     # calls of about a millisecond and more
    return {"decode_rope": lambda: leg_decode_rope(args.steps, args.warmup, base_ms),
            "decode_per_agent": lambda: leg_decode_per_agent(args.steps, args.warmup, base_ms),
            "decode_qkvo_r4": lambda: leg_decode_qkvo_r4(args.steps, args.warmup),
            "naive_decode": lambda: leg_naive_decode(slow, 3, base_ms, pcpu),
            "prefill_rope": lambda: leg_prefill_rope(mid, 3),
            "prefill_paged": lambda: leg_prefill_paged(
                mid, 3, extra.get("prefill_rope", {}).get("ms_per_call")),
            "paged_decode": lambda: leg_paged_decode(mid, 3),
            "naive_prefill": lambda: leg_naive_prefill(
                mid, 3, extra.get("prefill_rope", {}).get("ms_per_call")),
            "naive_paged_decode": lambda: leg_naive_paged_decode(
                slow, 2, extra.get("paged_decode", {}).get("ms_per_call")),
            "workload1_fp32": lambda: leg_workload1_fp32(args.steps, 10),
            "agent_scaling": lambda: leg_agent_scaling(max(20, args.steps // 2), 5, pcpu),
            "lr_build": lambda: leg_lr_build(args.steps, 10),
            "prelr_step": lambda: leg_prelr_step(1, 1),
            "ceilings": lambda: leg_ceilings(args.steps, 3)}


ALL_LEGS = ("workload1_fp32,agent_scaling,decode_rope,decode_qkvo_r4,decode_per_agent,naive_decode,"
            "prefill_rope,prefill_paged,naive_prefill,paged_decode,naive_paged_decode,lr_build,"
            "prelr_step,ceilings")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets of the primary leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra legs")
    ap.add_argument("--extra", default=ALL_LEGS, help="comma-separated extra legs to run")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the primary leg's oracle timing (the extra legs keep theirs)")
    ap.add_argument("--no-oracle", action="store_true",
                    help="skip every oracle timing and parity check (profiling runs)")
    ap.add_argument("--no-primary", action="store_true",
                    help="skip the primary leg (profiling runs of single extra legs)")
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
    global CHECK
    CHECK = not args.no_oracle

    if args.no_primary:
        done = {}
        legs = _extra_legs(args, None, None, done)
        for name in [x for x in args.extra.split(",") if x]:
            _log(f"extra (alone): {name}")
            done[name] = legs[name]()
            print(json.dumps({name: done[name]}), flush=True)
        return

    _log("primary: decode, 4 shared contexts x 8192 tokens, 16 requests")
    # exactly --warmup untimed calls before the --steps timed ones
    case, ms, call_us, nbytes, got, _ = run_decode(args.steps, args.warmup, args.sets, min_warm_s=0.0)
    gbs = nbytes / (ms * 1e-3) / 1e9
    value = case.n_req / (ms * 1e-3)
    _log(f"primary: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s, {value:.0f} tokens/s")
    cpu = cpu1 = par = None
    if CHECK and not args.no_cpu_baseline:
        _log("primary: cpu baseline (oracle)")
        cpu, cpu1, par = primary_cpu_baselines(case, got)
    primary_cpu = cpu if cpu else _cpu(None, "tokens/s", "not measured in this run")

    extra = {}
    if not args.no_extra:
        legs = _extra_legs(args, ms, primary_cpu, extra)
        for name in [x for x in args.extra.split(",") if x]:
            fn = legs[name]
            _log(f"extra: {name}")
            t0 = time.perf_counter()
            try:
                extra[name] = fn()
                rl = extra[name].get("roofline")
                _log(f"extra: {name}: {extra[name]['value']:.4g} {extra[name]['unit']}"
                     + (f", {rl['frac'] * 100:.1f}% of peak" if rl else "")
                     + f" ({time.perf_counter() - t0:.0f} s)")
            except lra.LraError as e:
                extra[name] = {"error": str(e)}
                _log(f"extra: {name}: {e}")
            torch.cuda.empty_cache()

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
        "roofline": _roofline("primary", "hbm", gbs, nbytes),
        "cpu_baseline": cpu,
        "cpu_baseline_1core": cpu1,
        "parity": par,
        "call_us": call_us,
        "kernel_sources_sha256": kernel_sources_sha(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
