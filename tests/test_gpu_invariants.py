"""Structural invariants of the method checked on the GPU path: properties that hold at
any size and need no oracle arithmetic.

- GQA equals MHA with each KV head (and its B column block) repeated for its query heads,
  bit for bit (decode at equal KV chunks).
- B = 0 is plain attention: compared with torch's scaled_dot_product_attention run in
  float64 on the CPU from the same bf16 bits.
- Softmax rows sum to one: V_base = 1 and B_v = 0 give outputs of one (prefill, with and
  without RoPE on the adapter key).
- Swapping two agents' B swaps their outputs, and the output is affine in B_v (prefill).
"""
import dataclasses
import os

import numpy as np
import pytest

import workloads as w
from gpu_helpers import BF16_MAX_ABS, BF16_REL_L2, DecodeDev, PrefillDev, host, metrics

pytestmark = pytest.mark.gpu

ONE_ULP_AT_1 = 2.0 ** -7  # bf16 spacing just above 1.0


def _repeat_b(b, h_kv, d, g):
    """[n_agents, r, H_kv*d] -> [n_agents, r, H_kv*g*d]: KV head h's block for each of its g query heads."""
    n, r, _ = b.shape
    return np.ascontiguousarray(np.repeat(b.reshape(n, r, h_kv, d), g, axis=2).reshape(n, r, h_kv * g * d))


def _identical(a, b, what):
    """Two GPU results of the same rows, packed differently into the kernels' row tiles:
    each row's arithmetic (its MFMA elements, softmax state and merge order) does not depend
    on the row's position in a tile, so the bits agree."""
    ma, rel = metrics(a, b)
    print(f"[invariant] {what}: max-abs {ma:.2e} rel-L2 {rel:.2e} bit-identical {np.array_equal(a, b)}", flush=True)
    assert np.array_equal(a, b), f"{what}: max-abs {ma:.3e}, rel-L2 {rel:.3e}"


@pytest.mark.parametrize("chunk", ["512", "2048"])
def test_decode_gqa_equals_repeated_heads_mha(chunk):
    case = w.make_decode(61, dtype="bf16", ctx_lens=[3000, 777, 5000], reqs=[(0, 0), (0, 1), (1, 2), (2, 0), (2, 2)],
                         n_agents=3, h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="gqa")
    g = case.h_q // case.h_kv
    mha = dataclasses.replace(case, h_kv=case.h_q, k_pool=np.ascontiguousarray(np.repeat(case.k_pool, g, axis=1)),
                              v_pool=np.ascontiguousarray(np.repeat(case.v_pool, g, axis=1)),
                              b_k=_repeat_b(case.b_k, case.h_kv, case.d, g),
                              b_v=_repeat_b(case.b_v, case.h_kv, case.d, g), name="mha")
    old = os.environ.get("LRA_DECODE_CHUNK")
    os.environ["LRA_DECODE_CHUNK"] = chunk  # the same KV chunks (hence merge order) on both sides
    try:
        got_gqa = host(DecodeDev(case).run())
        got_mha = host(DecodeDev(mha).run())
    finally:
        if old is None:
            del os.environ["LRA_DECODE_CHUNK"]
        else:
            os.environ["LRA_DECODE_CHUNK"] = old
    _identical(got_gqa, got_mha, f"decode GQA g=4 vs MHA, chunk {chunk}")


@pytest.mark.parametrize("rope", [False, True])
def test_prefill_gqa_equals_repeated_heads_mha(rope):
    case = w.make_prefill(62, dtype="bf16", kv_len=600, q_len=70, req_agents=[1, 0], n_agents=2, h_q=16,
                          h_kv=4, d=128, r=16, rope_theta=500000.0 if rope else None, name="gqa")
    g = case.h_q // case.h_kv
    mha = dataclasses.replace(case, h_kv=case.h_q, k_base=np.ascontiguousarray(np.repeat(case.k_base, g, axis=0)),
                              v_base=np.ascontiguousarray(np.repeat(case.v_base, g, axis=0)),
                              b_k=_repeat_b(case.b_k, case.h_kv, case.d, g),
                              b_v=_repeat_b(case.b_v, case.h_kv, case.d, g), name="mha")
    _identical(host(PrefillDev(case).run()), host(PrefillDev(mha).run()), f"prefill GQA g=4 vs MHA, rope {rope}")


def _sdpa64(q, k, v, causal_offset=None):
    """float64 torch SDPA on the CPU.  q [H_q, n, d], k/v [H_q, L, d]; causal_offset = the
    absolute position of query row 0 (bottom-right alignment), None for no mask."""
    import torch
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    mask = None
    if causal_offset is not None:
        n, L = q.shape[1], k.shape[1]
        mask = torch.arange(L)[None, :] <= (causal_offset + torch.arange(n))[:, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).numpy()


def _assert_bar(got, ref, what):
    ma, rel = metrics(got, ref)
    print(f"[invariant] {what}: max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)
    assert ma <= BF16_MAX_ABS and rel <= BF16_REL_L2, f"{what}: max-abs {ma:.3e}, rel-L2 {rel:.3e}"


def test_decode_zero_b_is_sdpa():
    import torch
    case = w.make_decode(63, dtype="bf16", ctx_lens=[1500, 40, 2600], reqs=[(0, 0), (0, 1), (1, 1), (2, 0)],
                         n_agents=2, h_q=32, h_kv=8, d=128, r=16, shuffle=True, q_sigma=4.0, name="b=0")
    d = DecodeDev(case)
    got = host(d.run(b_k=torch.zeros_like(d.b_k), b_v=torch.zeros_like(d.b_v)))
    g = case.h_q // case.h_kv
    kp, vp = w.widen(case.k_pool), w.widen(case.v_pool)  # [n_pages, H_kv, page, d]
    for i in range(case.n_req):
        c = int(case.req_ctx[i])
        L = int(case.ctx_len[c])
        pages = case.block_table[c, :(L + case.page - 1) // case.page]
        k = np.concatenate([kp[p] for p in pages], axis=1)[:, :L]  # [H_kv, L, d]
        v = np.concatenate([vp[p] for p in pages], axis=1)[:, :L]
        ref = _sdpa64(w.widen(case.q[i])[:, None, :], np.repeat(k, g, axis=0), np.repeat(v, g, axis=0))[:, 0]
        _assert_bar(got[i], ref, f"decode request {i} (context {c}, {L} keys), B = 0 vs SDPA")


@pytest.mark.parametrize("rope", [False, True])
def test_prefill_zero_b_is_sdpa(rope):
    import torch
    case = w.make_prefill(64, dtype="bf16", kv_len=900, q_len=150, req_agents=[0, 1], n_agents=2, h_q=32,
                          h_kv=8, d=128, r=16, rope_theta=500000.0 if rope else None, q_sigma=4.0, name="b=0")
    d = PrefillDev(case)
    got = host(d.run(b_k=torch.zeros_like(d.b_k), b_v=torch.zeros_like(d.b_v)))  # [n_req, q_len, H_q, d]
    g = case.h_q // case.h_kv
    k = np.repeat(w.widen(case.k_base), g, axis=0)
    v = np.repeat(w.widen(case.v_base), g, axis=0)
    for i in range(case.n_req):
        q = w.widen(case.q[i]).transpose(1, 0, 2)  # [H_q, q_len, d]
        ref = _sdpa64(q, k, v, causal_offset=case.kv_len - case.q_len).transpose(1, 0, 2)
        _assert_bar(got[i], ref, f"prefill request {i}, rope {rope}, B = 0 vs SDPA (causal)")


@pytest.mark.parametrize("rope", [False, True])
def test_prefill_rows_sum_to_one(rope):
    """V_base = 1 and B_v = 0: every output is sum(p) / sum(p) = 1, whatever the scores
    (which keep B_k and, with RoPE, the rotated adapter key)."""
    import torch
    import attention_shared_base_amd as lra
    case = w.make_prefill(65, dtype="bf16", kv_len=1000, q_len=333, req_agents=[2, 0, 1], n_agents=3, h_q=32,
                          h_kv=8, d=128, r=16, rope_theta=500000.0 if rope else None, q_sigma=4.0, name="ones")
    d = PrefillDev(case)
    got = host(lra.prefill(d.q, d.agent, d.k, torch.ones_like(d.v), d.lk, d.lv, d.b_k, torch.zeros_like(d.b_v),
                           rope_cos=d.cos, rope_sin=d.sin))
    err = float(np.max(np.abs(got - 1.0)))
    print(f"[invariant] prefill rows sum to one, rope {rope}: max |O - 1| {err:.2e}", flush=True)
    assert err <= ONE_ULP_AT_1


def test_prefill_agent_swap_and_bv_affinity():
    import torch
    case = w.make_prefill(66, dtype="bf16", kv_len=700, q_len=90, req_agents=[0, 1], n_agents=2, h_q=32,
                          h_kv=8, d=128, r=16, rope_theta=500000.0, name="swap")
    case.q[1] = case.q[0]
    d = PrefillDev(case)
    base = host(d.run())
    swapped = host(d.run(b_k=d.b_k.flip(0).contiguous(), b_v=d.b_v.flip(0).contiguous()))
    assert np.array_equal(base[0], swapped[1]) and np.array_equal(base[1], swapped[0])
    o0 = host(d.run(b_v=torch.zeros_like(d.b_v)))
    o2 = host(d.run(b_v=(d.b_v.float() * 2).to(torch.bfloat16)))
    dev_ = np.max(np.abs((o2 - base) - (base - o0)))
    print(f"[invariant] prefill affine in B_v: max deviation {dev_:.2e}", flush=True)
    assert dev_ < 3 * 2.0 ** -8 * max(1.0, np.max(np.abs(o2)))
