"""GPU checks of the paged serving loop: appending tokens to the page pools
(lra_cache_append), chunked prefill over a paged context read in place
(lra_attn_prefill_paged) or through a staging copy (lra_attn_prefill_paged_staged),
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


def _paged_context(case, n_pages, seed, poison=True):
    """The case's context in shuffled pages of device pools.  With ``poison`` every
    slot no key of the context occupies (unused pages, the tail of the last page)
    holds NaN, and the block-table row carries out-of-range ids past the context's
    blocks: neither may reach the output."""
    import torch
    n_blk = (case.kv_len + 15) // 16
    ids = np.random.default_rng(seed).permutation(n_pages)[:n_blk]
    kp, lkp = w.paginate(case.k_base, case.l_k, ids, n_pages, 16)
    vp, lvp = w.paginate(case.v_base, case.l_v, ids, n_pages, 16)
    pools = [dev(x) for x in w.decode_device_layout(kp, vp, lkp, lvp)]
    row = ids.astype(np.int32)
    if poison:
        k, v, lk, lv = pools
        unused = torch.from_numpy(np.setdiff1d(np.arange(n_pages), ids)).to("cuda")
        for t in pools:
            t[unused] = float("nan")
        last, tail = int(ids[-1]), case.kv_len - 16 * (n_blk - 1)
        k[last, :, :, tail:, :] = float("nan")
        v[last, :, :, tail:] = float("nan")
        lk[last, tail:, :] = float("nan")
        lv[last, :, tail:] = float("nan")
        row = np.concatenate([row, np.array([-7, n_pages + 100, 1 << 30, -1], np.int32)])
    return pools, torch.from_numpy(row).to("cuda")


PAGED_CASES = [
    # rope, h_q, h_kv, d, r, kv_len, q_len
    (False, 32, 8, 128, 16, 777, 100),
    (True, 32, 8, 128, 16, 777, 100),
    (False, 8, 8, 64, 8, 640, 64),       # kv_len a multiple of the 64-key tile
    (True, 8, 8, 64, 8, 640, 64),
    (True, 32, 8, 128, 4, 300, 300),     # the whole context is new
    (False, 32, 8, 128, 4, 1040, 90),    # kv_len a multiple of the page, not of the tile
    (False, 16, 4, 128, 32, 1000, 37),
    (True, 32, 8, 128, 32, 1000, 37),
    (True, 32, 1, 64, 16, 33, 1),        # one token, 32 query heads per KV head
    (True, 16, 8, 64, 32, 129, 65),
]


@pytest.mark.parametrize("rope,h_q,h_kv,d,r,kv_len,q_len", PAGED_CASES,
                         ids=[f"{'rope ' if c[0] else ''}g{c[1] // c[2]} d{c[3]} r{c[4]} kv{c[5]} q{c[6]}"
                              for c in PAGED_CASES])
def test_prefill_paged_equals_contiguous(rope, h_q, h_kv, d, r, kv_len, q_len):
    """Paged prefill reading the pages in place = contiguous prefill over the same context
    (same bits), also with NaN in every slot outside the context and junk block-table
    entries past it; the staged path gives the same bits; both match the oracle."""
    import torch
    import attention_shared_base_amd as lra
    case = w.make_prefill(63 + kv_len, dtype="bf16", kv_len=kv_len, q_len=q_len, req_agents=[1, 0],
                          n_agents=2, h_q=h_q, h_kv=h_kv, d=d, r=r,
                          rope_theta=500000.0 if rope else None, b_sigma=0.2, name="paged prefill")
    n_pages = (kv_len + 15) // 16 + 11
    d_ = PrefillDev(case)
    ref_gpu = d_.run()
    print(f"[paged prefill rope={rope} g{h_q // h_kv} d{d} r{r} kv{kv_len} q{q_len}] ", end="", flush=True)
    for poison in (False, True):
        pools, table = _paged_context(case, n_pages, 5 + kv_len, poison=poison)
        got = lra.prefill_paged(d_.q, d_.agent, *pools, table, kv_len, d_.b_k, d_.b_v,
                                rope_cos=d_.cos, rope_sin=d_.sin)
        assert torch.equal(got, ref_gpu), f"direct paged != contiguous (poison={poison})"
        if not poison:  # the staged copy reads whole pages, NaN tails included
            st = lra.prefill_paged_staged(d_.q, d_.agent, *pools, table, kv_len, d_.b_k, d_.b_v,
                                          rope_cos=d_.cos, rope_sin=d_.sin)
            assert torch.equal(st, ref_gpu), "staged paged != contiguous"
    ma, rel = assert_parity(host(got), oracle_prefill(case), "bf16", "paged prefill")
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


@pytest.mark.parametrize("rope,r", [(False, 16), (True, 16), (True, 4), (False, 32)])
def test_prefill_paged_per_agent_lr(rope, r):
    """One LR pool per agent ([n_agents, n_pages, 16, r] / [.., r, 16]) through the same block
    table, with and without RoPE on the adapter key: equals the contiguous per-agent prefill
    bit for bit, and the oracle."""
    import torch
    import attention_shared_base_amd as lra
    n_ag, kv_len = 3, 700
    case = w.make_prefill(91, dtype="bf16", kv_len=kv_len, q_len=90, req_agents=[2, 0, 1, 2],
                          n_agents=n_ag, h_q=32, h_kv=8, d=128, r=r, b_sigma=0.2,
                          rope_theta=500000.0 if rope else None, name="per-agent paged prefill")
    rng = np.random.default_rng(92)
    lk = np.stack([w.f32_to_bf16_bits(rng.standard_normal(case.l_k.shape).astype(np.float32))
                   for _ in range(n_ag)])
    lv = np.stack([w.f32_to_bf16_bits(rng.standard_normal(case.l_v.shape).astype(np.float32))
                   for _ in range(n_ag)])
    n_pages = 50
    ids = np.random.default_rng(93).permutation(n_pages)[:(kv_len + 15) // 16]
    kp, _ = w.paginate(case.k_base, case.l_k, ids, n_pages, 16)
    vp, _ = w.paginate(case.v_base, case.l_v, ids, n_pages, 16)
    lkps, lvps = [], []
    for a in range(n_ag):
        _, lkp = w.paginate(case.k_base, lk[a], ids, n_pages, 16)
        _, lvp = w.paginate(case.v_base, lv[a], ids, n_pages, 16)
        k, v, lkd, lvd = w.decode_device_layout(kp, vp, lkp, lvp)
        lkps.append(lkd)
        lvps.append(lvd)
    d_ = PrefillDev(case)
    table = torch.from_numpy(ids.astype(np.int32)).to("cuda")
    got = lra.prefill_paged(d_.q, d_.agent, dev(k), dev(v), dev(np.stack(lkps)), dev(np.stack(lvps)),
                            table, kv_len, d_.b_k, d_.b_v, rope_cos=d_.cos, rope_sin=d_.sin)
    assert torch.equal(got, d_.run(lk=dev(lk), lv=dev(lv)))
    ma, rel = assert_parity(host(got), oracle_prefill(case, l_k=w.widen(lk), l_v=w.widen(lv)), "bf16",
                            "per-agent paged prefill")
    print(f"[per-agent paged prefill rope={rope} r{r}] max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)


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
