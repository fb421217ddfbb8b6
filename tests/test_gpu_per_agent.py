"""GPU parity with one LR cache per agent (LRAgent §3 BaseShared; PReCache PreLRShared
with per-agent A): decode, prefill and the naive baseline read each request's own agent's
L_k / L_v, the cache append writes every agent's pools, and one LR-build call produces
every agent's cache, X [A_1 .. A_n].  Against the float64 oracle."""
import os

import numpy as np
import pytest

import workloads as w
from gpu_helpers import DecodeDev, PrefillDev, assert_parity, dev, host, oracle_decode, oracle_prefill

pytestmark = pytest.mark.gpu


def _per_agent_pools(case, n_agents, seed):
    """Per-agent logical LR pools shaped like the case's shared ones (own draws)."""
    rng = np.random.default_rng(seed)
    conv = (lambda x: w.f32_to_bf16_bits(x)) if case.dtype == "bf16" else (lambda x: x)
    lk = np.stack([conv(rng.standard_normal(case.lk_pool.shape).astype(np.float32))
                   for _ in range(n_agents)])
    lv = np.stack([conv(rng.standard_normal(case.lv_pool.shape).astype(np.float32))
                   for _ in range(n_agents)])
    return lk, lv


def _device_lr(lk, lv):
    """Per-agent logical pools -> [n_agents, n_pages, 16, r] / [n_agents, n_pages, r, 16]."""
    return dev(np.ascontiguousarray(lk)), dev(np.ascontiguousarray(lv.transpose(0, 1, 3, 2)))


def _decode_case(label, h_q, h_kv, d, r, lens, rpc, dtype="bf16", n_agents=4, seed=81):
    reqs = [(c, (c + i) % n_agents) for c in range(len(lens)) for i in range(rpc)]
    case = w.make_decode(seed, dtype=dtype, ctx_lens=lens, reqs=reqs, n_agents=n_agents, h_q=h_q,
                         h_kv=h_kv, d=d, r=r, shuffle=True, b_sigma=0.2, name=label)
    lk, lv = _per_agent_pools(case, n_agents, seed + 1)
    return case, lk, lv


CASES = [
    # label, h_q, h_kv, d, r, ctx_lens, requests per context
    ("g4 d128 r16 four agents per context", 32, 8, 128, 16, [3000, 1, 1025], 4),
    ("g1 d64 r8 six requests (two row groups)", 8, 8, 64, 8, [300, 17], 6),
    ("g8 d128 r32", 16, 2, 128, 32, [2049, 64], 3),
    ("g4 d128 r4", 32, 8, 128, 4, [1500, 40], 4),
]


@pytest.mark.parametrize("label,h_q,h_kv,d,r,lens,rpc", CASES, ids=[c[0] for c in CASES])
def test_decode_per_agent_lr(label, h_q, h_kv, d, r, lens, rpc):
    case, lk, lv = _decode_case(label, h_q, h_kv, d, r, lens, rpc)
    dd = DecodeDev(case)
    lk_d, lv_d = _device_lr(lk, lv)
    got = host(dd.run(lk=lk_d, lv=lv_d))
    case.lk_pool, case.lv_pool = lk, lv
    ref = oracle_decode(case)
    print(f"[per-agent decode] {label}: ", end="", flush=True)
    ma, rel = assert_parity(got, ref, "bf16", label)
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


def test_decode_per_agent_identical_caches_equal_shared():
    """Every agent holding the same LR cache gives the shared-cache result bit for bit."""
    case, _, _ = _decode_case("identical", 32, 8, 128, 16, [2500, 700], 4)
    dd = DecodeDev(case)
    shared = host(dd.run())
    n_ag = case.b_k.shape[0]
    lk_d = dd.lk.unsqueeze(0).expand(n_ag, *dd.lk.shape).contiguous()
    lv_d = dd.lv.unsqueeze(0).expand(n_ag, *dd.lv.shape).contiguous()
    assert np.array_equal(host(dd.run(lk=lk_d, lv=lv_d)), shared)


def test_decode_per_agent_fp32_and_persistent():
    case, lk, lv = _decode_case("fp32 per agent", 8, 2, 128, 16, [45, 300, 1], 2, dtype="f32")
    dd = DecodeDev(case)
    lk_d, lv_d = _device_lr(lk, lv)
    got = host(dd.run(lk=lk_d, lv=lv_d))
    case.lk_pool, case.lv_pool = lk, lv
    assert_parity(got, oracle_decode(case), "f32", "fp32 per agent")
    # bf16, long uneven contexts, persistent workgroups and chunk sizes
    case, lk, lv = _decode_case("persistent per agent", 32, 8, 128, 16, [9000, 300, 4500], 4)
    dd = DecodeDev(case)
    lk_d, lv_d = _device_lr(lk, lv)
    case.lk_pool, case.lv_pool = lk, lv
    ref = oracle_decode(case)
    try:
        for chunk, per in (("512", "1"), ("1024", "0")):
            os.environ["LRA_DECODE_CHUNK"] = chunk
            os.environ["LRA_DECODE_PERSISTENT"] = per
            assert_parity(host(dd.run(lk=lk_d, lv=lv_d)), ref, "bf16", f"chunk {chunk} persistent {per}")
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_per_agent_lr(dtype):
    n_ag = 3
    case = w.make_prefill(83, dtype=dtype, kv_len=700, q_len=90, req_agents=[2, 0, 1, 2],
                          n_agents=n_ag, h_q=32, h_kv=8, d=128, r=16, b_sigma=0.2,
                          name=f"per-agent prefill {dtype}")
    rng = np.random.default_rng(84)
    conv = (lambda x: w.f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x)
    lk = np.stack([conv(rng.standard_normal(case.l_k.shape).astype(np.float32)) for _ in range(n_ag)])
    lv = np.stack([conv(rng.standard_normal(case.l_v.shape).astype(np.float32)) for _ in range(n_ag)])
    got = host(PrefillDev(case).run(lk=dev(lk), lv=dev(lv)))
    ref = oracle_prefill(case, l_k=w.widen(lk), l_v=w.widen(lv))
    ma, rel = assert_parity(got, ref, dtype, f"per-agent prefill {dtype}")
    print(f"[per-agent prefill {dtype}] max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


def test_lr_build_multi_a():
    """One call builds four agents' LR caches; each equals X A_a (oracle, fp64) within bf16
    rounding and equals the single-agent build bit for bit."""
    import torch
    import attention_shared_base_amd as lra
    import oracle
    n_ag, n_tok, d_model, r, rows, off = 4, 1000, 4096, 16, 1200, 150
    rng = np.random.default_rng(85)
    x = w.f32_to_bf16_bits(rng.standard_normal((n_tok, d_model)).astype(np.float32))
    a_k = w.f32_to_bf16_bits((rng.standard_normal((n_ag, r, d_model)) / 64).astype(np.float32))
    a_v = w.f32_to_bf16_bits((rng.standard_normal((n_ag, r, d_model)) / 64).astype(np.float32))
    lk = torch.zeros((n_ag, rows, r), dtype=torch.bfloat16, device="cuda")
    lv = torch.zeros_like(lk)
    lra.lr_cache_build(dev(x), dev(a_k), dev(a_v), lk, lv, row_offset=off)
    got_k, got_v = host(lk), host(lv)
    for a in range(n_ag):
        ek, ev = oracle.lr_cache_build(w.widen(x), w.widen(a_k[a]).T, w.widen(a_v[a]).T)
        for got, e in ((got_k[a, off:off + n_tok], ek), (got_v[a, off:off + n_tok], ev)):
            # fp32 accumulation of 4096 products, one bf16 rounding
            assert np.max(np.abs(got - e) / (np.abs(e) + 1e-2)) < 2 ** -7
        assert np.all(got_k[a, :off] == 0) and np.all(got_k[a, off + n_tok:] == 0)
        one_k = torch.zeros((rows, r), dtype=torch.bfloat16, device="cuda")
        one_v = torch.zeros_like(one_k)
        lra.lr_cache_build(dev(x), dev(a_k[a]), dev(a_v[a]), one_k, one_v, row_offset=off)
        assert torch.equal(one_k, lk[a]) and torch.equal(one_v, lv[a])


def test_append_per_agent_pools():
    """Appending with one LR row set per agent (n_lr = 3) writes every agent's pools in the
    page layout bit for bit, and leaves the base pools as the shared append does."""
    import torch
    import attention_shared_base_amd as lra
    n_ag, n_tok, n_pages, r = 3, 200, 20, 16
    case = w.make_prefill(95, dtype="bf16", kv_len=n_tok, q_len=1, req_agents=[0], n_agents=1,
                          h_q=32, h_kv=8, d=128, r=r, name="per-agent append")
    rng = np.random.default_rng(96)
    lk = np.stack([w.f32_to_bf16_bits(rng.standard_normal((n_tok, r)).astype(np.float32))
                   for _ in range(n_ag)])
    lv = np.stack([w.f32_to_bf16_bits(rng.standard_normal((n_tok, r)).astype(np.float32))
                   for _ in range(n_ag)])
    ids = np.random.default_rng(97).permutation(n_pages)[:(n_tok + 15) // 16]
    tok = np.arange(n_tok)
    slots = torch.from_numpy((ids[tok // 16] * 16 + tok % 16).astype(np.int64)).to("cuda")
    z = dict(dtype=torch.bfloat16, device="cuda")
    kp, vp = torch.zeros((n_pages, 8, 16, 16, 8), **z), torch.zeros((n_pages, 8, 128, 16), **z)
    lkp, lvp = torch.zeros((n_ag, n_pages, 16, r), **z), torch.zeros((n_ag, n_pages, r, 16), **z)
    k_new = dev(np.ascontiguousarray(case.k_base.transpose(1, 0, 2)))
    v_new = dev(np.ascontiguousarray(case.v_base.transpose(1, 0, 2)))
    lra.cache_append(slots, k_new, v_new, dev(lk), dev(lv), kp, vp, lkp, lvp)
    for a in range(n_ag):
        kl, lkl = w.paginate(case.k_base, lk[a], ids, n_pages, 16)
        vl, lvl = w.paginate(case.v_base, lv[a], ids, n_pages, 16)
        want = w.decode_device_layout(kl, vl, lkl, lvl)
        for got, ref, name in ((kp, want[0], "K"), (vp, want[1], "V"), (lkp[a], want[2], "L_k"),
                               (lvp[a], want[3], "L_v")):
            g = got.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(g, ref), f"{name} agent {a}"


def test_naive_decode_per_agent_pools():
    """The naive baseline with one LR pool per agent expands each request with its own
    agent's L rows: equal to the method's per-agent decode within bf16 rounding, and to
    the oracle."""
    import attention_shared_base_amd as lra
    case, lk, lv = _decode_case("naive per agent", 32, 8, 128, 16, [1500, 333], 4)
    dd = DecodeDev(case)
    lk_d, lv_d = _device_lr(lk, lv)
    method = host(dd.run(lk=lk_d, lv=lv_d))
    naive = host(lra.naive_decode(dd.q, dd.crs, dd.agent, dd.k, dd.v, lk_d, lv_d, dd.bt, dd.clen,
                                  dd.b_k, dd.b_v, max_req_per_ctx=dd.max_req_per_ctx,
                                  max_ctx_len=dd.max_ctx_len))
    case.lk_pool, case.lv_pool = lk, lv
    ref = oracle_decode(case)
    ma, rel = assert_parity(naive, ref, "bf16", "naive per agent")
    assert_parity(method, ref, "bf16", "method per agent")
    print(f"[per-agent naive decode] max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


ROPE_CASES = [
    # label, h_q, h_kv, d, r, ctx_lens, requests per context
    ("rope g4 d128 r16 four agents per context", 32, 8, 128, 16, [3000, 1, 1025], 4),
    ("rope g8 d128 r32", 16, 2, 128, 32, [2049, 64], 3),
    ("rope g1 d64 r8 six requests (two row groups)", 8, 8, 64, 8, [300, 17], 6),
    ("rope g4 d128 r4", 32, 8, 128, 4, [1500, 40], 4),
]


@pytest.mark.parametrize("label,h_q,h_kv,d,r,lens,rpc", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_decode_rope_per_agent_lr(label, h_q, h_kv, d, r, lens, rpc):
    """RoPE on the adapter key with one LR cache per agent (BaseShared under RoPE, LRAgent
    App. D.1): each request's rotated key term is rebuilt from its own agent's L_k."""
    import torch
    from gpu_helpers import DELTA_REL_L2, metrics
    case, lk, lv = _decode_case(label, h_q, h_kv, d, r, lens, rpc)
    dd = DecodeDev(case)
    lk_d, lv_d = _device_lr(lk, lv)
    got = host(dd.run(lk=lk_d, lv=lv_d, rope_theta=500000.0))
    case.lk_pool, case.lv_pool = lk, lv
    ref = oracle_decode(case, rope_theta=500000.0)
    print(f"[per-agent rope decode] {label}: ", end="", flush=True)
    ma, rel = assert_parity(got, ref, "bf16", label)
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)
    # the adapter's contribution on its own, and the rotation's: the unrotated per-agent
    # result misses the oracle's adapter delta by far more than the rotated one
    zb = dict(b_k=torch.zeros_like(dd.b_k), b_v=torch.zeros_like(dd.b_v))
    got0 = host(dd.run(lk=lk_d, lv=lv_d, rope_theta=500000.0, **zb))
    ref0 = oracle_decode(case, zero_b=True, rope_theta=500000.0)
    _, rel_d = metrics(got - got0, ref - ref0)
    assert rel_d <= DELTA_REL_L2, f"adapter delta rel-L2 {rel_d:.3e}"
    plain = host(dd.run(lk=lk_d, lv=lv_d))
    assert metrics(plain - got0, ref - ref0)[1] > 4 * rel_d


def test_decode_rope_per_agent_identical_caches_equal_shared():
    """Every agent holding the same LR cache gives the shared-cache RoPE result bit for bit
    (same rebuild, same rounding, same value products)."""
    case, _, _ = _decode_case("rope identical", 32, 8, 128, 16, [2500, 700], 4)
    dd = DecodeDev(case)
    shared = host(dd.run(rope_theta=500000.0))
    n_ag = case.b_k.shape[0]
    lk_d = dd.lk.unsqueeze(0).expand(n_ag, *dd.lk.shape).contiguous()
    lv_d = dd.lv.unsqueeze(0).expand(n_ag, *dd.lv.shape).contiguous()
    assert np.array_equal(host(dd.run(lk=lk_d, lv=lv_d, rope_theta=500000.0)), shared)
