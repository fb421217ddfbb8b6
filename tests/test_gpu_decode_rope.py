"""GPU parity of paged decode with RoPE on the adapter key term (lra_attn_decode with
rope tables) against the float64 oracle.

With RoPE the key adapter term is rebuilt per request at head dimension, rotated by
its key's position and rounded once to bf16 before the score MFMA (LRAgent App. D.1);
the base key stays exact.  That rounding is relative 2^-9 on a term of size ~|B_k|,
far inside the standard bars, which every case here keeps.
"""
import os

import numpy as np
import pytest

import workloads as w
from gpu_helpers import (DELTA_REL_L2, DecodeDev, PrefillDev, assert_parity, host, metrics,
                         oracle_decode)

pytestmark = pytest.mark.gpu

THETA = 500000.0


def _check(case, theta=THETA, requests=None, label="", d=None):
    d = d or DecodeDev(case)
    got = host(d.run(rope_theta=theta))
    ref = oracle_decode(case, requests=requests, rope_theta=theta)
    sel = slice(None) if requests is None else list(requests)
    print(f"[decode rope] {label or case.name}: ", end="", flush=True)
    ma, rel = assert_parity(got[sel], ref[sel], case.dtype, label or case.name)
    print(f"max-abs {ma:.2e} rel-L2 {rel:.2e} |O|inf {np.max(np.abs(ref[sel])):.3f}", flush=True)
    return d, got, ref


def test_cfg2_shape_decode_rope_full():
    """16 requests over 4 shared 8192-token contexts, RoPE theta 5e5 on the adapter key."""
    case = w.config2()
    d, got, ref = _check(case, label="cfg2 shapes + rope")
    import torch
    got0 = host(d.run(b_k=torch.zeros_like(d.b_k), b_v=torch.zeros_like(d.b_v), rope_theta=THETA))
    ref0 = oracle_decode(case, zero_b=True, rope_theta=THETA)
    _, rel = metrics(got - got0, ref - ref0)
    assert rel <= DELTA_REL_L2, f"adapter delta rel-L2 {rel:.3e}"
    # the rotation is visible at this size: the unrotated result differs from the oracle
    plain = host(d.run())
    assert metrics(plain - got0, ref - ref0)[1] > 4 * rel


SMALL = [
    # (label, h_q, h_kv, d, r, ctx_lens, reqs_per_ctx, b_sigma)
    ("g4 d128 r16 ragged", 32, 8, 128, 16, [1, 17, 33, 100, 257, 1000], 2, 0.3),
    ("g1 d64 r8", 8, 8, 64, 8, [5, 16, 31, 129], 3, 0.3),
    ("g8 d128 r32", 16, 2, 128, 32, [15, 64, 200, 2049], 1, 0.3),
    ("g4 d64 r16 multi row-group", 4, 1, 64, 16, [300, 48], 6, 0.3),
    ("g2 d128 r8", 8, 4, 128, 8, [2, 1500], 5, 0.3),
    ("g16 d64 r32", 16, 1, 64, 32, [77, 4096], 1, 0.3),
    ("g1 d128 r32 sixteen requests", 4, 4, 128, 32, [700], 16, 0.3),
    # rank 4 with RoPE on the adapter key: the pages' qkvo setting (App. D.1)
    ("g4 d128 r4 qkvo rank", 32, 8, 128, 4, [33, 700, 1100], 2, 0.3),
    ("g1 d64 r4", 8, 8, 64, 4, [5, 129], 3, 0.3),
]


@pytest.mark.parametrize("label,h_q,h_kv,d,r,lens,rpc,bs", SMALL, ids=[s[0] for s in SMALL])
def test_decode_rope_small_shuffled(label, h_q, h_kv, d, r, lens, rpc, bs):
    n_agents = 3
    reqs = [(c, (c + i) % n_agents) for c in range(len(lens)) for i in range(rpc)]
    case = w.make_decode(41, dtype="bf16", ctx_lens=lens, reqs=reqs, n_agents=n_agents, h_q=h_q,
                         h_kv=h_kv, d=d, r=r, shuffle=True, b_sigma=bs, name=label)
    _check(case, theta=10000.0)



def test_decode_rope_long_chunks_high_frequencies():
    """4096-token chunks (32 steps per wavefront: the keys' cos / sin advanced by angle addition
    31 times) at theta 1e4, whose fastest pair turns 128 rad per step, with a large adapter term
    (B ~ N(0, 0.3^2)): the whole result and the adapter's own contribution against the oracle,
    whose tables are computed per position."""
    import torch
    reqs = [(c, c % 3) for c in range(3) for _ in range(2)]
    case = w.make_decode(57, dtype="bf16", ctx_lens=[8191, 4096, 6000], reqs=reqs, n_agents=3, h_q=32,
                         h_kv=8, d=128, r=16, shuffle=True, b_sigma=0.3, name="rope long chunks")
    try:
        os.environ["LRA_DECODE_CHUNK"] = "4096"
        d, got, ref = _check(case, theta=10000.0, label="rope 4096-token chunks theta 1e4")
        got0 = host(d.run(b_k=torch.zeros_like(d.b_k), b_v=torch.zeros_like(d.b_v), rope_theta=10000.0))
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
    ref0 = oracle_decode(case, zero_b=True, rope_theta=10000.0)
    _, rel = metrics(got - got0, ref - ref0)
    assert rel <= DELTA_REL_L2, f"adapter delta rel-L2 {rel:.3e}"

def test_decode_rope_fp32():
    reqs = [(0, 0), (0, 1), (1, 1), (2, 0)]
    case = w.make_decode(43, dtype="f32", ctx_lens=[1, 45, 300], reqs=reqs, n_agents=2, h_q=8,
                         h_kv=2, d=128, r=32, shuffle=True, b_sigma=0.3, name="fp32 rope")
    _check(case, theta=10000.0)


def test_decode_rope_zero_bk_equals_plain():
    """With B_k = 0 the rotated adapter key is zero: RoPE and no-RoPE decode agree exactly."""
    import torch
    reqs = [(0, 0), (0, 1), (1, 1), (2, 0)]
    case = w.make_decode(47, dtype="bf16", ctx_lens=[3000, 77, 1025], reqs=reqs, n_agents=2,
                         h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="zero bk")
    d = DecodeDev(case)
    zk = torch.zeros_like(d.b_k)
    a = host(d.run(b_k=zk, rope_theta=THETA))
    b = host(d.run(b_k=zk))
    assert np.array_equal(a, b)


def test_decode_rope_equals_last_prefill_row():
    """Decode of the last new token = last row of the RoPE prefill over the same caches."""
    case = w.make_prefill(49, dtype="bf16", kv_len=1234, q_len=50, req_agents=[0, 1, 2],
                          n_agents=3, h_q=32, h_kv=8, d=128, r=16, rope_theta=THETA,
                          b_sigma=0.2, name="decode-vs-prefill rope")
    pre = host(PrefillDev(case).run())
    n_pages = (1234 + 15) // 16
    ids = np.random.default_rng(1).permutation(n_pages)
    kp, lkp = w.paginate(case.k_base, case.l_k, ids, n_pages, 16)
    vp, lvp = w.paginate(case.v_base, case.l_v, ids, n_pages, 16)
    dec = w.DecodeCase(dtype="bf16", h_q=32, h_kv=8, d=128, r=16, page=16,
                       q=np.ascontiguousarray(case.q[:, -1]),
                       req_ctx=np.zeros(3, np.int32), req_agent=case.req_agent,
                       ctx_len=np.array([1234], np.int32),
                       block_table=ids.astype(np.int32)[None, :], k_pool=kp, v_pool=vp,
                       lk_pool=lkp, lv_pool=lvp, b_k=case.b_k, b_v=case.b_v)
    out = host(DecodeDev(dec).run(rope_theta=THETA))
    # the prefill rounds K' = K_base + rot(dK) to bf16, the decode only rot(dK)
    assert np.max(np.abs(out - pre[:, -1])) < 2e-2
    assert metrics(out, pre[:, -1])[1] < 1e-2


@pytest.mark.skip(reason="the RoPE decode's persistent (chunk-queue) form is switched off: a GPU "
                         "memory fault was observed with it (rank 32, 512-token chunks) and its cause "
                         "has not been found; the library never launches it")
def test_decode_rope_persistent_queue():
    """Persistent workgroups with RoPE on the adapter key (not launched; see the reason)."""


def test_decode_rope_splits():
    """Chunk sizes with RoPE (one workgroup per chunk; the RoPE decode never runs its
    persistent form, also when asked to): same rows, workspace back to zero."""
    import torch
    import attention_shared_base_amd as lra
    reqs = [(c, c % 3) for c in range(5) for _ in range(2)] + [(5, 1)]
    case = w.make_decode(53, dtype="bf16", ctx_lens=[3000, 1, 9000, 0, 4500, 700], reqs=reqs,
                         n_agents=3, h_q=32, h_kv=8, d=128, r=32, shuffle=True, b_sigma=0.2,
                         name="rope splits")
    d = DecodeDev(case)
    live = [i for i, (c, _) in enumerate(reqs) if c != 3]
    ref = oracle_decode(case, requests=live, rope_theta=THETA)
    outs = []
    try:
        os.environ["LRA_DECODE_CHUNK"] = "256"  # the most chunks: the largest workspace
        n_ws = lra.decode_workspace_size(n_q_heads=32, n_kv_heads=8, head_dim=128, rank=32, dtype=1,
                                         n_req=len(reqs), n_ctx=6, max_req_per_ctx=d.max_req_per_ctx,
                                         max_ctx_len=d.max_ctx_len)
        ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
        for chunk, per in (("512", "0"), ("512", "0"), ("256", "0"), ("4096", "0")):
            os.environ["LRA_DECODE_CHUNK"] = chunk
            os.environ["LRA_DECODE_PERSISTENT"] = per
            print(f"[decode rope] chunk {chunk} persistent {per}", flush=True)
            outs.append(host(d.run(workspace=ws, rope_theta=THETA)))
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)
    for o in outs:
        assert_parity(o[live], ref[live], "bf16", "rope splits")
        assert np.all(o[[6, 7]] == 0.0)
    assert np.array_equal(outs[0], outs[1])  # the same call twice: the same bits
