"""GPU checks of the paged serving loop: appending tokens to the page pools
(lra_cache_append), chunked prefill over a paged context (lra_attn_prefill_paged)
and decode after a decode-time append, against the float64 oracle."""
import numpy as np
import pytest

import workloads as w
from gpu_helpers import DecodeDev, PrefillDev, assert_parity, dev, host, oracle_decode, oracle_prefill

pytestmark = pytest.mark.gpu


def _pools_for(case_kv_len, h_kv, d, r, n_pages):
    import torch
    z = dict(dtype=torch.bfloat16, device="cuda")
    return (torch.zeros((n_pages, h_kv, d // 8, 16, 8), **z), torch.zeros((n_pages, h_kv, d, 16), **z),
            torch.zeros((n_pages, 16, r), **z), torch.zeros((n_pages, r, 16), **z))


def _append(case, pools, ids, t0, t1):
    """Append tokens t0..t1-1 of a PrefillCase's caches through the slot mapping."""
    import torch
    import attention_shared_base_amd as lra
    tok = np.arange(t0, t1)
    slots = torch.from_numpy((ids[tok // 16] * 16 + tok % 16).astype(np.int64)).to("cuda")
    k_new = dev(np.ascontiguousarray(case.k_base[:, t0:t1].transpose(1, 0, 2)))
    v_new = dev(np.ascontiguousarray(case.v_base[:, t0:t1].transpose(1, 0, 2)))
    lra.cache_append(slots, k_new, v_new, dev(case.l_k[t0:t1]), dev(case.l_v[t0:t1]), *pools)


@pytest.mark.parametrize("r", [16, 4])
def test_append_builds_the_page_layout(r):
    """Appending a whole context token range by range gives exactly the pools the
    layout helper builds (bit-exact), including a partial last page and skipped slots."""
    import torch
    import attention_shared_base_amd as lra
    case = w.make_prefill(61, dtype="bf16", kv_len=1000, q_len=8, req_agents=[0], n_agents=1,
                          h_q=32, h_kv=8, d=128, r=r, name="append")
    n_pages = 70
    ids = np.random.default_rng(3).permutation(n_pages)[:63]
    pools = _pools_for(1000, 8, 128, r, n_pages)
    for t0, t1 in ((0, 300), (300, 999), (999, 1000)):  # prefill chunks, then one decode token
        _append(case, pools, ids, t0, t1)
    # a negative slot is skipped
    neg = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    junk = torch.ones((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    lra.cache_append(neg, junk, junk, junk[:, 0, :r].contiguous(), junk[:, 0, :r].contiguous(), *pools)
    kp, lkp = w.paginate(case.k_base, case.l_k, ids, n_pages, 16)
    vp, lvp = w.paginate(case.v_base, case.l_v, ids, n_pages, 16)
    want = w.decode_device_layout(kp, vp, lkp, lvp)
    for got, ref, name in zip(pools, want, ("K", "V", "L_k", "L_v")):
        g = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(g, ref), name


@pytest.mark.parametrize("rope", [False, True])
def test_prefill_paged_equals_contiguous(rope):
    """Paged prefill = contiguous prefill over the same context (same bits), and the oracle."""
    import torch
    import attention_shared_base_amd as lra
    case = w.make_prefill(63, dtype="bf16", kv_len=777, q_len=100, req_agents=[1, 0], n_agents=2,
                          h_q=32, h_kv=8, d=128, r=16, rope_theta=500000.0 if rope else None,
                          b_sigma=0.2, name="paged prefill")
    n_pages = 60
    ids = np.random.default_rng(5).permutation(n_pages)[:49]
    kp, lkp = w.paginate(case.k_base, case.l_k, ids, n_pages, 16)
    vp, lvp = w.paginate(case.v_base, case.l_v, ids, n_pages, 16)
    pools = [dev(x) for x in w.decode_device_layout(kp, vp, lkp, lvp)]
    d = PrefillDev(case)
    table = torch.from_numpy(ids.astype(np.int32)).to("cuda")
    got = lra.prefill_paged(d.q, d.agent, *pools, table, 777, d.b_k, d.b_v, rope_cos=d.cos,
                            rope_sin=d.sin)
    ref_gpu = d.run()
    assert torch.equal(got, ref_gpu)
    ref = oracle_prefill(case)
    print(f"[paged prefill rope={rope}] ", end="", flush=True)
    ma, rel = assert_parity(host(got), ref, "bf16", "paged prefill")
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


def test_serving_loop_append_prefill_decode():
    """A context grows through the pools: 500 cached tokens, a 64-token chunk appended and
    prefilled by two agents, then one decode-time append and a decode step for each."""
    import torch
    import attention_shared_base_amd as lra
    L0, C = 500, 64
    full = w.make_prefill(67, dtype="bf16", kv_len=L0 + C + 1, q_len=C + 1, req_agents=[0, 1],
                          n_agents=2, h_q=32, h_kv=8, d=128, r=16, b_sigma=0.2, name="loop")
    n_pages = 48
    ids = np.random.default_rng(7).permutation(n_pages)[:(L0 + C + 1 + 15) // 16]
    pools = _pools_for(L0 + C + 1, 8, 128, 16, n_pages)
    table = torch.from_numpy(ids.astype(np.int32)).to("cuda")
    _append(full, pools, ids, 0, L0)          # the cached context
    _append(full, pools, ids, L0, L0 + C)     # the new chunk (its LR rows built earlier)
    chunk = w.PrefillCase(dtype="bf16", h_q=32, h_kv=8, d=128, r=16,
                          q=np.ascontiguousarray(full.q[:, :C]), req_agent=full.req_agent,
                          k_base=np.ascontiguousarray(full.k_base[:, :L0 + C]),
                          v_base=np.ascontiguousarray(full.v_base[:, :L0 + C]),
                          l_k=np.ascontiguousarray(full.l_k[:L0 + C]),
                          l_v=np.ascontiguousarray(full.l_v[:L0 + C]), b_k=full.b_k, b_v=full.b_v)
    got = lra.prefill_paged(dev(chunk.q), dev(chunk.req_agent), *pools, table, L0 + C,
                            dev(chunk.b_k), dev(chunk.b_v))
    assert_parity(host(got), oracle_prefill(chunk), "bf16", "loop prefill")
    _append(full, pools, ids, L0 + C, L0 + C + 1)  # decode-time append of the next token
    n = L0 + C + 1
    dec = w.DecodeCase(dtype="bf16", h_q=32, h_kv=8, d=128, r=16, page=16,
                       q=np.ascontiguousarray(full.q[:, C]), req_ctx=np.zeros(2, np.int32),
                       req_agent=full.req_agent, ctx_len=np.array([n], np.int32),
                       block_table=ids.astype(np.int32)[None, :],
                       k_pool=np.zeros((1,)), v_pool=np.zeros((1,)), lk_pool=np.zeros((1,)),
                       lv_pool=np.zeros((1,)), b_k=full.b_k, b_v=full.b_v)
    out = lra.decode(dev(dec.q), dev(dec.ctx_req_start()), dev(dec.req_agent), *pools, table[None, :],
                     dev(dec.ctx_len), dev(dec.b_k), dev(dec.b_v), max_req_per_ctx=2, max_ctx_len=n)
    kp, lkp = w.paginate(full.k_base, full.l_k, ids, n_pages, 16)
    vp, lvp = w.paginate(full.v_base, full.l_v, ids, n_pages, 16)
    dec.k_pool, dec.v_pool, dec.lk_pool, dec.lv_pool = kp, vp, lkp, lvp
    assert_parity(host(out), oracle_decode(dec), "bf16", "loop decode")
