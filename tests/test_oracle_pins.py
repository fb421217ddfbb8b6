"""Pins for the float64 oracle (CPU only).

Nothing on the pages prints a worked numeric example, so the oracle is pinned by
what the mathematics fixes: pure-Python brute force, B = 0 reducing to plain
attention (checked against torch's SDPA routine), the reordering identity and
the RoPE barrier stated in LRAgent (arXiv 2602.01053v2, §3 and App. B / App.
D.1), softmax normalisation, closed-form special cases and the hand-derived
fixtures in tests/golden/.  The mutation tests at the end plant plausible
mistakes in the oracle and check that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from oracle.brute import brute_attention, brute_matmul

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, *, n_rows=3, h_q=2, h_kv=1, d=4, r=2, kv_len=6, b_sigma=0.5):
    rng = np.random.default_rng(seed)
    return dict(
        q=rng.standard_normal((n_rows, h_q, d)),
        k_base=rng.standard_normal((h_kv, kv_len, d)),
        v_base=rng.standard_normal((h_kv, kv_len, d)),
        l_k=rng.standard_normal((kv_len, r)),
        l_v=rng.standard_normal((kv_len, r)),
        b_k=b_sigma * rng.standard_normal((r, h_kv * d)),
        b_v=b_sigma * rng.standard_normal((r, h_kv * d)),
    )


def tolist(c):
    return {k: v.tolist() for k, v in c.items()}


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("mode", ["decode", "causal", "causal_rope"])
def test_brute_force_matches_oracle(seed, mode):
    h_q, h_kv = (2, 1) if seed % 2 == 0 else (4, 2)
    d = 4
    c = rand_case(seed, h_q=h_q, h_kv=h_kv, d=d, r=2, kv_len=7, n_rows=3)
    kv_len = 7
    if mode == "decode":
        q_pos = [kv_len - 1] * 3
    else:
        q_pos = [kv_len - 3 + i for i in range(3)]
    theta = 10000.0 if mode == "causal_rope" else None
    rope = ref.rope_tables(kv_len, d, theta) if theta else None
    got = ref.attention_materialised(**c, q_pos=q_pos, rope=rope)
    want = np.array(brute_attention(**tolist(c), q_pos=q_pos, rope_theta=theta))
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_brute_force_lr_build():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 6))
    a_k = rng.standard_normal((6, 2))
    a_v = rng.standard_normal((6, 2))
    lk, lv = ref.lr_cache_build(x, a_k, a_v)
    assert np.max(np.abs(lk - np.array(brute_matmul(x.tolist(), a_k.tolist())))) < 1e-13
    assert np.max(np.abs(lv - np.array(brute_matmul(x.tolist(), a_v.tolist())))) < 1e-13


# ----------------------------------------------------------------------------- (a) B = 0

@pytest.mark.parametrize("causal", [False, True])
def test_b_zero_is_plain_attention_sdpa(causal):
    torch = pytest.importorskip("torch")
    c = rand_case(11, n_rows=5, h_q=4, h_kv=2, d=8, r=3, kv_len=9)
    c["b_k"][:] = 0
    c["b_v"][:] = 0
    kv_len, n_rows = 9, 5
    q_pos = (np.arange(n_rows) + kv_len - n_rows) if causal else np.full(n_rows, kv_len - 1)
    got = ref.attention_materialised(**c, q_pos=q_pos)
    g = 2
    q = torch.from_numpy(c["q"]).permute(1, 0, 2)                    # [H_q, n, d]
    k = torch.from_numpy(c["k_base"]).repeat_interleave(g, dim=0)    # [H_q, L, d]
    v = torch.from_numpy(c["v_base"]).repeat_interleave(g, dim=0)
    mask = torch.from_numpy(ref.causal_visible(q_pos, kv_len))
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    want = want.permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) < 1e-13


# ----------------------------------------------------------------------------- (b) reordering

@pytest.mark.parametrize("seed", range(4))
def test_reordered_and_augmented_equal_materialised(seed):
    c = rand_case(100 + seed, n_rows=6, h_q=8, h_kv=2, d=16, r=4, kv_len=33, b_sigma=0.3)
    q_pos = np.arange(6) + 33 - 6
    m = ref.attention_materialised(**c, q_pos=q_pos)
    assert rel_err(ref.attention_reordered(**c, q_pos=q_pos), m) < 1e-12
    assert rel_err(ref.attention_augmented(**c, q_pos=q_pos), m) < 1e-12


def test_rope_barrier_blocks_score_reordering():
    """With RoPE on the adapter key term the reordered score form is NOT the definition."""
    c = rand_case(5, n_rows=4, h_q=2, h_kv=1, d=8, r=2, kv_len=20, b_sigma=1.0)
    q_pos = np.arange(4) + 16
    rope = ref.rope_tables(20, 8, 10000.0)
    rotated = ref.attention_materialised(**c, q_pos=q_pos, rope=rope)
    reordered = ref.attention_reordered(**c, q_pos=q_pos)
    assert np.max(np.abs(rotated - reordered)) > 1e-3
    # value side is unaffected by the rotation: with B_k = 0 both forms agree again
    c["b_k"][:] = 0
    rotated = ref.attention_materialised(**c, q_pos=q_pos, rope=rope)
    assert rel_err(ref.attention_reordered(**c, q_pos=q_pos), rotated) < 1e-12


# ----------------------------------------------------------------------------- (c) normalisation

def test_softmax_rows_sum_to_one():
    c = rand_case(21, n_rows=7, h_q=4, h_kv=2, d=8, r=2, kv_len=12)
    q_pos = np.arange(7) + 5
    _, p = ref.attention_materialised(**c, q_pos=q_pos, return_probs=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-12
    vis = ref.causal_visible(q_pos, 12)
    assert np.all(p[:, ~vis] == 0.0)


def test_constant_values_give_constant_output():
    c = rand_case(22, n_rows=4, h_q=4, h_kv=2, d=8, r=2, kv_len=12)
    c["v_base"][:] = 1.0
    c["b_v"][:] = 0.0
    out = ref.attention_materialised(**c, q_pos=np.arange(4) + 8)
    assert np.max(np.abs(out - 1.0)) < 1e-14


# ----------------------------------------------------------------------------- closed forms

def test_single_key_returns_its_adapted_value():
    c = rand_case(31, n_rows=1, h_q=2, h_kv=1, d=4, r=2, kv_len=1)
    out = ref.attention_materialised(**c)
    v0 = c["v_base"][0, 0] + c["l_v"][0] @ c["b_v"][:, 0:4]
    assert np.max(np.abs(out[0, 0] - v0)) < 1e-15 and np.max(np.abs(out[0, 1] - v0)) < 1e-15


def test_zero_query_averages_visible_values():
    c = rand_case(32, n_rows=3, h_q=2, h_kv=1, d=4, r=2, kv_len=10)
    c["q"][:] = 0
    q_pos = np.array([3, 6, 9])
    out = ref.attention_materialised(**c, q_pos=q_pos)
    v = c["v_base"][0] + c["l_v"] @ c["b_v"]
    for i, p in enumerate(q_pos):
        assert np.max(np.abs(out[i, 0] - v[:p + 1].mean(0))) < 1e-14


def test_outlier_key_dominates():
    # A strongly aligned key late in the stream: the running max must move to it.
    c = rand_case(33, n_rows=1, h_q=1, h_kv=1, d=4, r=2, kv_len=64, b_sigma=0.0)
    c["k_base"] *= 0.01
    c["q"][0, 0] = [30.0, 0, 0, 0]
    c["k_base"][0, 50] = [2.0, 0, 0, 0]
    out = ref.attention_materialised(**c, scale=1.0)
    assert np.max(np.abs(out[0, 0] - c["v_base"][0, 50])) < 1e-20 + 1e-12 * 64


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((50, 16))
    cos, sin = ref.rope_tables(50, 16, 500000.0)
    y = ref.rope_rotate_half(x, cos, sin)
    assert np.all(y[0] == x[0])
    assert np.max(np.abs(np.linalg.norm(y, axis=1) - np.linalg.norm(x, axis=1))) < 1e-12


def test_rope_relative_position():
    """<R_m x, R_n y> depends only on n - m (the defining RoPE property)."""
    rng = np.random.default_rng(42)
    d = 8
    x = rng.standard_normal(d)
    y = rng.standard_normal(d)
    cos, sin = ref.rope_tables(40, d, 10000.0)

    def rot(v, p):
        return ref.rope_rotate_half(v[None], cos[p:p + 1], sin[p:p + 1])[0]

    for m, n in [(3, 10), (13, 20), (0, 7)]:
        assert abs(rot(x, m) @ rot(y, n) - x @ rot(y, n - m)) < 1e-12
    # and the pairing is rotate-half: for d=2 the frequency is 1 and R_1 e0 = (cos 1, sin 1)
    c2, s2 = ref.rope_tables(2, 2, 123.0)
    assert np.allclose(ref.rope_rotate_half(np.array([[1.0, 0.0]]), c2[1:], s2[1:]),
                       [[math.cos(1.0), math.sin(1.0)]], atol=1e-16)
    # frequencies: theta^(-2i/d)
    assert np.allclose(ref.rope_inv_freq(8, 500000.0), [500000.0 ** (-2 * i / 8) for i in range(4)],
                       rtol=1e-15)


def test_causal_row_ignores_future_keys():
    c = rand_case(51, n_rows=4, h_q=2, h_kv=1, d=4, r=2, kv_len=10)
    q_pos = np.arange(4) + 6
    base = ref.attention_materialised(**c, q_pos=q_pos)
    c["k_base"][0, 9] += 100.0
    c["l_v"][9] += 5.0
    moved = ref.attention_materialised(**c, q_pos=q_pos)
    assert np.all(moved[:3] == base[:3])
    assert np.max(np.abs(moved[3] - base[3])) > 1e-3


def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "closed_form_two_keys.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        arr = {k: np.array(cs[k], dtype=np.float64)
               for k in ("q", "k_base", "v_base", "l_k", "l_v", "b_k", "b_v")}
        kv_len = arr["k_base"].shape[1]
        d = arr["q"].shape[2]
        rope = ref.rope_tables(kv_len, d, cs["rope_theta"]) if cs["rope_theta"] else None
        got = ref.attention_materialised(**arr, q_pos=cs["q_pos"], scale=cs["scale"], rope=rope)
        assert np.max(np.abs(got - np.array(cs["expected"]))) < 1e-14, cs["name"]
        bf = brute_attention(**{k: v.tolist() for k, v in arr.items()}, q_pos=cs["q_pos"],
                             scale=cs["scale"], rope_theta=cs["rope_theta"])
        assert np.max(np.abs(np.array(bf) - np.array(cs["expected"]))) < 1e-14, cs["name"]


# ----------------------------------------------------------------------------- paging

def test_gather_pages_inverts_paginate():
    from workloads import paginate
    rng = np.random.default_rng(61)
    kv = rng.standard_normal((2, 45, 4))
    lr = rng.standard_normal((45, 3))
    ids = rng.permutation(5)
    kvp, lrp = paginate(kv, lr, ids, 5, 16)
    # only three of the five pool pages are used by this context
    g_kv, g_lr = ref.gather_pages(kvp, lrp, ids, 45)
    assert np.array_equal(g_kv, kv) and np.array_equal(g_lr, lr)


def test_decode_equals_last_prefill_row():
    from workloads import paginate
    rng = np.random.default_rng(62)
    h_q, h_kv, d, r, L = 4, 2, 8, 2, 37
    c = rand_case(63, n_rows=5, h_q=h_q, h_kv=h_kv, d=d, r=r, kv_len=L)
    pre = ref.prefill(c["q"][None], [0], c["k_base"], c["v_base"], c["l_k"], c["l_v"],
                      c["b_k"][None], c["b_v"][None])
    ids = rng.permutation(3)
    kp, lkp = paginate(c["k_base"], c["l_k"], ids, 3, 16)
    vp, lvp = paginate(c["v_base"], c["l_v"], ids, 3, 16)
    dec = ref.decode_paged(c["q"][-1:], [0], [0], kp, vp, lkp, lvp, ids[None], [L],
                           c["b_k"][None], c["b_v"][None])
    assert np.max(np.abs(dec[0] - pre[0, -1])) < 1e-14


def test_prefill_rows_subset_matches_full():
    c = rand_case(64, n_rows=8, h_q=2, h_kv=1, d=4, r=2, kv_len=20)
    full = ref.prefill(c["q"][None], [0], c["k_base"], c["v_base"], c["l_k"], c["l_v"],
                       c["b_k"][None], c["b_v"][None], row_chunk=3)
    sub = ref.prefill(c["q"][None], [0], c["k_base"], c["v_base"], c["l_k"], c["l_v"],
                      c["b_k"][None], c["b_v"][None], rows=[0, 5, 7])
    assert np.array_equal(sub[0], full[0, [0, 5, 7]])


# ----------------------------------------------------------------------------- mutation checks

def _pins_catch(monkeypatch, name, mutant):
    """Run the brute-force and identity pins against a mutated oracle; True if one fails."""
    monkeypatch.setattr(ref, name, mutant)
    failed = False
    for seed in range(3):
        c = rand_case(seed, h_q=4, h_kv=2, d=4, r=2, kv_len=7, n_rows=3)
        q_pos = [4, 5, 6]
        for theta in (None, 10000.0):
            rope = ref.rope_tables(7, 4, theta) if theta else None
            got = ref.attention_materialised(**c, q_pos=q_pos, rope=rope)
            want = np.array(brute_attention(**tolist(c), q_pos=q_pos, rope_theta=theta))
            failed |= bool(np.max(np.abs(got - want)) > 1e-12)
    return failed


def test_pins_catch_planted_mistakes(monkeypatch):
    orig_rot = ref.rope_rotate_half
    orig_sm = ref.softmax_two_pass
    orig_vis = ref.causal_visible

    def rot_sign(x, cos, sin):  # rotation the wrong way round
        return orig_rot(x, cos, -sin)

    def rot_interleaved(x, cos, sin):  # wrong pairing: (2i, 2i+1)
        y = x.copy()
        y[..., 0::2] = x[..., 0::2] * cos - x[..., 1::2] * sin
        y[..., 1::2] = x[..., 1::2] * cos + x[..., 0::2] * sin
        return y

    def sm_unnormalised(s):
        m = np.max(s, axis=-1, keepdims=True)
        return np.exp(s - m)

    def vis_strict(q_pos, kv_len):  # excludes the row's own key
        return orig_vis(q_pos, kv_len) & ~(np.arange(kv_len)[None, :] == np.asarray(q_pos)[:, None])

    with monkeypatch.context() as mp:
        assert _pins_catch(mp, "rope_rotate_half", rot_sign)
    with monkeypatch.context() as mp:
        assert _pins_catch(mp, "rope_rotate_half", rot_interleaved)
    with monkeypatch.context() as mp:
        assert _pins_catch(mp, "softmax_two_pass", sm_unnormalised)
    with monkeypatch.context() as mp:
        assert _pins_catch(mp, "causal_visible", vis_strict)
    assert ref.softmax_two_pass is orig_sm


def test_pins_catch_wrong_head_slice_and_transpose():
    """Plausible index mistakes in the B slice / operand orientation differ from brute force."""
    c = rand_case(3, h_q=4, h_kv=2, d=4, r=2, kv_len=7, n_rows=3)
    q_pos = [4, 5, 6]
    want = np.array(brute_attention(**tolist(c), q_pos=q_pos))
    # head 1 reading head 0's slice of B
    bad = dict(c)
    bad["b_k"] = np.concatenate([c["b_k"][:, :4], c["b_k"][:, :4]], axis=1)
    bad["b_v"] = np.concatenate([c["b_v"][:, :4], c["b_v"][:, :4]], axis=1)
    assert np.max(np.abs(ref.attention_materialised(**bad, q_pos=q_pos) - want)) > 1e-6
    # dropping the key-side adapter term
    bad = dict(c)
    bad["b_k"] = np.zeros_like(c["b_k"])
    assert np.max(np.abs(ref.attention_materialised(**bad, q_pos=q_pos) - want)) > 1e-6
    # grouping query heads interleaved (hq % H_kv) instead of contiguous (hq // g)
    q_perm = c["q"][:, [0, 2, 1, 3], :]
    bad = dict(c)
    bad["q"] = q_perm
    got = ref.attention_materialised(**bad, q_pos=q_pos)[:, [0, 2, 1, 3], :]
    assert np.max(np.abs(got - want)) > 1e-6


def test_decode_rope_matches_brute_force():
    """Paged decode with RoPE on the adapter key (LRAgent App. D.1) against the
    pure-Python brute force: two contexts of different lengths, shuffled pages,
    requests of two agents, the query at each context's last position."""
    from workloads import paginate
    rng = np.random.default_rng(65)
    h_q, h_kv, d, r, theta = 4, 2, 8, 2, 10000.0
    lens = [21, 35]
    n_pages = 6
    ids = rng.permutation(n_pages)
    table = np.array([ids[:3], ids[3:]])
    kp = np.zeros((n_pages, h_kv, 16, d))
    vp = np.zeros_like(kp)
    lkp = np.zeros((n_pages, 16, r))
    lvp = np.zeros_like(lkp)
    ctxs = []
    for c, L in enumerate(lens):
        cs = rand_case(66 + c, n_rows=1, h_q=h_q, h_kv=h_kv, d=d, r=r, kv_len=L)
        k1, l1 = paginate(cs["k_base"], cs["l_k"], table[c], n_pages, 16)
        v1, l2 = paginate(cs["v_base"], cs["l_v"], table[c], n_pages, 16)
        for blk in range((L + 15) // 16):
            pid = table[c][blk]
            kp[pid], vp[pid], lkp[pid], lvp[pid] = k1[pid], v1[pid], l1[pid], l2[pid]
        ctxs.append(cs)
    q = rng.standard_normal((3, h_q, d))
    b_k = 0.5 * rng.standard_normal((2, r, h_kv * d))
    b_v = 0.5 * rng.standard_normal((2, r, h_kv * d))
    req_ctx, req_agent = [0, 1, 1], [1, 0, 1]
    rope = ref.rope_tables(max(lens), d, theta)
    got = ref.decode_paged(q, req_ctx, req_agent, kp, vp, lkp, lvp, table, lens, b_k, b_v,
                           rope=rope)
    for i in range(3):
        cs = ctxs[req_ctx[i]]
        L = lens[req_ctx[i]]
        want = brute_attention(q[i][None].tolist(), cs["k_base"].tolist(), cs["v_base"].tolist(),
                               cs["l_k"].tolist(), cs["l_v"].tolist(), b_k[req_agent[i]].tolist(),
                               b_v[req_agent[i]].tolist(), q_pos=[L - 1], rope_theta=theta)
        assert np.max(np.abs(got[i] - np.array(want[0]))) < 1e-12
    # the rotation matters here: without it the result moves
    plain = ref.decode_paged(q, req_ctx, req_agent, kp, vp, lkp, lvp, table, lens, b_k, b_v)
    assert np.max(np.abs(plain - got)) > 1e-3


def test_per_agent_lr_caches_match_brute_force():
    """BaseShared (LRAgent §3): each agent has its own A, hence its own LR cache.  Decode and
    prefill with per-agent LR pools equal the brute force run with each request's own L;
    with one cache repeated for every agent they equal the shared-cache result."""
    from workloads import paginate
    rng = np.random.default_rng(71)
    h_q, h_kv, d, r, L, n_ag = 4, 2, 8, 2, 29, 3
    c = rand_case(72, n_rows=1, h_q=h_q, h_kv=h_kv, d=d, r=r, kv_len=L)
    lk = rng.standard_normal((n_ag, L, r))
    lv = rng.standard_normal((n_ag, L, r))
    b_k = 0.5 * rng.standard_normal((n_ag, r, h_kv * d))
    b_v = 0.5 * rng.standard_normal((n_ag, r, h_kv * d))
    q = rng.standard_normal((3, h_q, d))
    agents = [2, 0, 1]
    ids = rng.permutation(2)
    kp, _ = paginate(c["k_base"], lk[0], ids, 2, 16)
    vp, _ = paginate(c["v_base"], lv[0], ids, 2, 16)
    lkp = np.stack([paginate(c["k_base"], lk[a], ids, 2, 16)[1] for a in range(n_ag)])
    lvp = np.stack([paginate(c["v_base"], lv[a], ids, 2, 16)[1] for a in range(n_ag)])
    dec = ref.decode_paged(q, [0, 0, 0], agents, kp, vp, lkp, lvp, ids[None], [L], b_k, b_v)
    pre = ref.prefill(q[:, None], agents, c["k_base"], c["v_base"], lk, lv, b_k, b_v)
    for i, a in enumerate(agents):
        want = np.array(brute_attention(q[i][None].tolist(), c["k_base"].tolist(),
                                        c["v_base"].tolist(), lk[a].tolist(), lv[a].tolist(),
                                        b_k[a].tolist(), b_v[a].tolist(), q_pos=[L - 1]))[0]
        assert np.max(np.abs(dec[i] - want)) < 1e-12
        assert np.max(np.abs(pre[i, 0] - want)) < 1e-12
    same = ref.decode_paged(q, [0, 0, 0], agents, kp, vp, np.stack([lkp[1]] * n_ag),
                            np.stack([lvp[1]] * n_ag), ids[None], [L], b_k, b_v)
    shared = ref.decode_paged(q, [0, 0, 0], agents, kp, vp, lkp[1], lvp[1], ids[None], [L], b_k, b_v)
    assert np.array_equal(same, shared)
