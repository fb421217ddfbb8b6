"""GPU parity of paged decode (lra_attn_decode) against the float64 oracle."""
import os

import numpy as np
import pytest

import workloads as w
from gpu_helpers import (DELTA_REL_L2, DecodeDev, assert_parity, host, metrics, oracle_decode)

pytestmark = pytest.mark.gpu


def _check(case, requests=None, label=""):
    d = DecodeDev(case)
    got = host(d.run())
    ref = oracle_decode(case, requests=requests)
    sel = slice(None) if requests is None else list(requests)
    print(f"[decode] {label or case.name}: ", end="", flush=True)
    ma, rel = assert_parity(got[sel], ref[sel], case.dtype, label or case.name)
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e} |O|inf {np.max(np.abs(ref[sel])):.3f}", flush=True)
    return d, got, ref


def test_cfg1_decode_fp32():
    dec, _ = w.config1()
    _check(dec)


def test_cfg2_decode_bf16_full():
    case = w.config2()
    d, got, ref = _check(case)
    # adapter contribution on its own (dropping the LR path would move rel-L2 ~0.2)
    import torch
    got0 = host(d.run(b_k=torch.zeros_like(d.b_k), b_v=torch.zeros_like(d.b_v)))
    ref0 = oracle_decode(case, zero_b=True)
    _, rel = metrics(got - got0, ref - ref0)
    assert rel <= DELTA_REL_L2, f"adapter delta rel-L2 {rel:.3e}"


def test_cfg2_decode_peaked_queries():
    # Q x 8: scores with sd ~ 8, so max-abs is a meaningful check as well
    case = w.make_decode(2, dtype="bf16", ctx_lens=[8192] * 4,
                         reqs=[(b // 4, b % 4) for b in range(16)], n_agents=4, h_q=32, h_kv=8,
                         d=128, r=16, q_sigma=8.0, name="cfg2 peaked (q sigma 8)")
    _check(case)


SMALL = [
    # (label, h_q, h_kv, d, r, ctx_lens, reqs_per_ctx)
    ("g4 d128 r16 ragged", 32, 8, 128, 16, [1, 17, 33, 100, 257, 1000], 2),
    ("g1 d64 r8", 8, 8, 64, 8, [5, 16, 31, 129], 3),
    ("g8 d128 r32", 16, 2, 128, 32, [15, 64, 200, 2049], 1),
    ("g4 d64 r16 multi row-group", 4, 1, 64, 16, [300, 48], 6),
    ("g2 d128 r8", 8, 4, 128, 8, [2, 1500], 5),
    ("g16 d64 r32", 16, 1, 64, 32, [77, 4096], 1),
    # rank 4: the query/key/value/output LoRA setting (LRAgent App. D.1)
    ("g4 d128 r4", 32, 8, 128, 4, [1, 17, 300, 1025, 2049], 2),
    ("g2 d64 r4", 8, 4, 64, 4, [50, 700], 3),
]


@pytest.mark.parametrize("label,h_q,h_kv,d,r,lens,rpc", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_shuffled(label, h_q, h_kv, d, r, lens, rpc):
    n_agents = 3
    reqs = [(c, (c + i) % n_agents) for c in range(len(lens)) for i in range(rpc)]
    case = w.make_decode(17, dtype="bf16", ctx_lens=lens, reqs=reqs, n_agents=n_agents, h_q=h_q,
                         h_kv=h_kv, d=d, r=r, shuffle=True, name=label)
    _check(case)


def test_decode_more_than_64_requests():
    """85 requests over 29 contexts of 3 (the row groups straddle request 64): past 64
    requests the kernel reads each group's agent ids from a table loaded at the group's
    first request instead of the one it fetches for requests 0..63."""
    lens = [(97 * c) % 700 + 1 for c in range(29)]
    reqs = [(c, (c + 2 * i) % 5) for c in range(29) for i in range(3)][:85]
    case = w.make_decode(43, dtype="bf16", ctx_lens=lens, reqs=reqs, n_agents=5, h_q=8, h_kv=2,
                         d=64, r=8, name="85 requests")
    d, _, ref = _check(case)
    # 512-token chunks (split-K merges), one workgroup per chunk and persistent workgroups
    try:
        os.environ["LRA_DECODE_CHUNK"] = "512"
        for per in ("0", "1"):
            os.environ["LRA_DECODE_PERSISTENT"] = per
            assert_parity(host(d.run()), ref, "bf16", f"85 requests, 512-token chunks, persistent={per}")
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)

@pytest.mark.parametrize("r", [32, 4])
def test_decode_fp32_ragged(r):
    reqs = [(0, 0), (0, 1), (1, 1), (2, 0)]
    case = w.make_decode(19, dtype="f32", ctx_lens=[1, 45, 300], reqs=reqs, n_agents=2, h_q=8,
                         h_kv=2, d=128, r=r, shuffle=True, b_sigma=0.1, name=f"fp32 ragged r{r}")
    _check(case)


FP32_EDGES = [(64, 4, False), (64, 16, True), (64, 32, False), (128, 8, True), (128, 16, False)]


@pytest.mark.parametrize("d,r,rope", FP32_EDGES, ids=[f"d{d} r{r}{' rope' if p else ''}" for d, r, p in FP32_EDGES])
def test_decode_fp32_chunk_edges(d, r, rope):
    """fp32 rows split over four wavefronts in 64-key chunks: contexts of 1, 63, 64, 65, 256
    (every wavefront one full chunk), 257 (the first wavefront a second one-key chunk) and
    1000 keys, at head-dim / rank pairs the other fp32 cases do not use."""
    ctx = [1, 63, 64, 65, 256, 257, 1000]
    reqs = [(c, c % 2) for c in range(len(ctx))]
    case = w.make_decode(29, dtype="f32", ctx_lens=ctx, reqs=reqs, n_agents=2, h_q=8, h_kv=2, d=d, r=r,
                         shuffle=True, b_sigma=0.2, name=f"fp32 chunk edges d{d} r{r} rope {rope}")
    theta = 10000.0 if rope else None
    got = host(DecodeDev(case).run(rope_theta=theta))
    ma, rel = assert_parity(got, oracle_decode(case, rope_theta=theta), "f32", case.name)
    print(f"[decode] {case.name}: max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


def test_decode_split_count_invariance():
    reqs = [(c, c % 3) for c in range(3) for _ in range(2)]
    case = w.make_decode(23, dtype="bf16", ctx_lens=[3000, 1111, 4096], reqs=reqs, n_agents=3,
                         h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="split invariance")
    d = DecodeDev(case)
    outs = []
    try:
        for chunk in ("256", "512", "1024", "2048", "4096"):
            os.environ["LRA_DECODE_CHUNK"] = chunk
            outs.append(host(d.run()))
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
    ref = oracle_decode(case)
    for o in outs:
        assert_parity(o, ref, "bf16", "split invariance")
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 4e-3


def test_decode_workspace_reuse_and_empty_context():
    import torch
    reqs = [(0, 0), (1, 1), (1, 0), (2, 1)]
    case = w.make_decode(29, dtype="bf16", ctx_lens=[5000, 0, 2500], reqs=reqs, n_agents=2,
                         h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="empty ctx")
    d = DecodeDev(case)
    import attention_shared_base_amd as lra
    ws = torch.zeros(lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1, n_req=4, n_ctx=3,
        max_req_per_ctx=d.max_req_per_ctx, max_ctx_len=d.max_ctx_len), dtype=torch.uint8,
        device="cuda")
    assert ws.numel() > 0
    a = host(d.run(workspace=ws))
    b = host(d.run(workspace=ws))
    c = host(d.run(workspace=ws))
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert np.all(a[1:3] == 0.0)  # requests on the empty context
    ref = oracle_decode(case, requests=[0, 3])
    assert_parity(a[[0, 3]], ref[[0, 3]], "bf16", "non-empty contexts")


def test_decode_row_sum_via_constant_values():
    import torch
    reqs = [(0, 0), (0, 1), (1, 1)]
    case = w.make_decode(31, dtype="bf16", ctx_lens=[999, 4000], reqs=reqs, n_agents=2, h_q=32,
                         h_kv=8, d=128, r=16, shuffle=True, name="row sum")
    case.v_pool[:] = w.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    d = DecodeDev(case)
    out = host(d.run(b_v=torch.zeros_like(d.b_v)))
    assert np.max(np.abs(out - 1.0)) <= 2.0 ** -7


def test_decode_agent_swap_and_bv_affinity():
    import torch
    reqs = [(0, 0), (0, 1)]
    case = w.make_decode(37, dtype="bf16", ctx_lens=[2222], reqs=reqs, n_agents=2, h_q=32,
                         h_kv=8, d=128, r=16, shuffle=True, name="agent swap")
    case.q[1] = case.q[0]
    d = DecodeDev(case)
    base = host(d.run())
    swapped = host(d.run(b_k=d.b_k.flip(0).contiguous(), b_v=d.b_v.flip(0).contiguous()))
    assert np.array_equal(base[0], swapped[1]) and np.array_equal(base[1], swapped[0])
    o0 = host(d.run(b_v=torch.zeros_like(d.b_v)))
    o2 = host(d.run(b_v=(d.b_v.float() * 2).to(torch.bfloat16)))
    # affine in B_v at fixed B_k (up to the bf16 rounding of the outputs)
    assert np.max(np.abs((o2 - base) - (base - o0))) < 3 * 2.0 ** -8 * max(1.0, np.max(np.abs(o2)))


def test_cfg4_paged_decode_all_requests():
    """Workload 4 at full size (32 contexts of 4096..65536 tokens in shuffled pages, 8
    agents, rank 32): every request's 32 rows against the oracle, plus each request's
    worst error reported."""
    case = w.config4()
    d, got, ref = _check(case, label="cfg4 all 32 requests")
    worst = max(range(len(case.req_agent)), key=lambda i: np.max(np.abs(got[i] - ref[i])))
    print(f"[decode] cfg4 worst request {worst} (len {case.ctx_len[case.req_ctx[worst]]}): "
          f"max-abs {np.max(np.abs(got[worst] - ref[worst])):.2e}", flush=True)
    for i in range(len(case.req_agent)):  # each request on its own at the same bar
        assert_parity(got[i:i + 1], ref[i:i + 1], "bf16", f"cfg4 request {i}")


def test_decode_persistent_queue():
    """Persistent workgroups pulling chunks from the workspace queue give the same rows as
    one workgroup per chunk, twice in a row on one workspace (the queue words return to 0)."""
    reqs = [(c, c % 3) for c in range(5) for _ in range(2)] + [(5, 1)]
    case = w.make_decode(31, dtype="bf16", ctx_lens=[3000, 1, 9000, 0, 4500, 700], reqs=reqs,
                         n_agents=3, h_q=32, h_kv=8, d=128, r=32, shuffle=True, name="persistent")
    import torch
    import attention_shared_base_amd as lra
    d = DecodeDev(case)
    live = [i for i, (c, _) in enumerate(reqs) if c != 3]  # context 3 is empty
    ref = oracle_decode(case, requests=live)
    outs = []
    try:
        os.environ["LRA_DECODE_CHUNK"] = "512"
        n_ws = lra.decode_workspace_size(n_q_heads=32, n_kv_heads=8, head_dim=128, rank=32, dtype=1,
                                         n_req=len(reqs), n_ctx=6, max_req_per_ctx=d.max_req_per_ctx,
                                         max_ctx_len=d.max_ctx_len)
        ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
        for per in ("0", "1", "1"):
            os.environ["LRA_DECODE_PERSISTENT"] = per
            outs.append(host(d.run(workspace=ws)))
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0  # counters and queue back at zero
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)
    for o in outs:
        assert_parity(o[live], ref[live], "bf16", "persistent")
        assert np.all(o[[6, 7]] == 0.0)  # requests on the empty context
    assert np.array_equal(outs[1], outs[2])
    assert np.max(np.abs(outs[1] - outs[0])) < 4e-3


@pytest.mark.parametrize("persistent", ["0", "1"])
def test_decode_context_longer_than_max_ctx_len(persistent):
    """A context length above max_ctx_len (device data the host cannot check) is cut to
    max_ctx_len: the call stays inside the workspace it was sized for, leaves the
    merge counters at zero, and a following valid call on the same workspace still
    matches the oracle."""
    import copy

    import torch
    import attention_shared_base_amd as lra
    reqs = [(0, 0), (0, 1), (1, 1), (2, 0)]
    case = w.make_decode(47, dtype="bf16", ctx_lens=[3000, 5000, 1500], reqs=reqs, n_agents=2,
                         h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="ctx_len > max_ctx_len")
    d = DecodeDev(case)
    cut = 2000
    try:
        os.environ["LRA_DECODE_CHUNK"] = "512"
        os.environ["LRA_DECODE_PERSISTENT"] = persistent
        n_ws = lra.decode_workspace_size(n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1,
                                         n_req=4, n_ctx=3, max_req_per_ctx=2, max_ctx_len=cut)
        ws = torch.zeros(lra.decode_workspace_size(
            n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1, n_req=4, n_ctx=3,
            max_req_per_ctx=2, max_ctx_len=d.max_ctx_len), dtype=torch.uint8, device="cuda")
        assert 0 < n_ws <= ws.numel()
        got = host(lra.decode(d.q, d.crs, d.agent, d.k, d.v, d.lk, d.lv, d.bt, d.clen, d.b_k, d.b_v,
                              max_req_per_ctx=2, max_ctx_len=cut, workspace=ws))
        torch.cuda.synchronize()
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0  # counters and queue at zero
        cut_case = copy.copy(case)
        cut_case.ctx_len = np.minimum(case.ctx_len, cut).astype(np.int32)
        assert_parity(got, oracle_decode(cut_case), "bf16", f"contexts cut to {cut}")
        full = host(d.run(workspace=ws))
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)
    assert_parity(full, oracle_decode(case), "bf16", "following valid call")


def test_prepared_decode_equals_decode():
    """lra.prepare_decode: the same launch as decode(), bit for bit, on every call; new
    contents of the same input tensors between calls are seen; RoPE tables pass through."""
    import torch
    import attention_shared_base_amd as lra
    case = w.make_decode(71, dtype="bf16", ctx_lens=[2500, 900], reqs=[(0, 0), (0, 1), (1, 1)], n_agents=2,
                         h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="prepared")
    d = DecodeDev(case)
    for theta in (None, 500000.0):
        ref = host(d.run(rope_theta=theta))
        cos, sin = d.rope(theta) if theta is not None else (None, None)
        out = torch.empty_like(d.q)
        call = lra.prepare_decode(d.q, d.crs, d.agent, d.k, d.v, d.lk, d.lv, d.bt, d.clen, d.b_k, d.b_v,
                                  max_req_per_ctx=d.max_req_per_ctx, max_ctx_len=d.max_ctx_len,
                                  rope_cos=cos, rope_sin=sin, out=out)
        for _ in range(3):
            assert np.array_equal(host(call()), ref)
        q_saved = d.q.clone()
        d.q.mul_(-1.0)
        flipped = host(d.run(rope_theta=theta))
        assert np.array_equal(host(call()), flipped) and not np.array_equal(flipped, ref)
        d.q.copy_(q_saved)
