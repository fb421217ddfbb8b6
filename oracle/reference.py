"""Float64 reference of multi-LoRA attention over shared base and low-rank caches.

TEST INFRASTRUCTURE — imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Shares no code with the HIP path.

Notation (LRAgent, arXiv 2602.01053v2, as summarised on paperlayer.ai and
gist.science):

* cache decomposition, App. A.3: ``Y_i = Y_base,i + dY_i`` with
  ``Y_base,i = X_i W0`` and ``dY_i = X_i A_i B_i``;
* BaseLRShared, §3: one shared down-projection ``A`` gives one LR cache
  ``Y_lr = X A`` (``[L, r]``) that all agents read; each agent applies its own
  up-projection ``B_i`` (``[r, d_out]``) at run time;
* App. B: one attention head sees ``V_lr`` of shape ``[L, r]`` and the
  up-projection ``B``; ``d_out = H_kv * d`` so head ``h`` uses the column
  slice ``B[:, h*d:(h+1)*d]`` (reading: the LR cache is shared by all KV heads
  because ``A`` maps ``d_model -> r``);
* App. D.1: with LoRA on the key projection the key must be rebuilt at head
  dimension *before* RoPE, because the position-dependent rotation blocks the
  associativity reordering used on the value side.

Everything here is the plain definition: the adapter term is materialised at
full head dimension, scores are formed explicitly, and the softmax is the
two-pass max/exp/sum form.  No blocking, streaming or reordering — except in
``attention_reordered`` / ``attention_augmented``, which exist only so tests
can pin the identities the pages state.

Layouts (all float64 on entry; callers widen bf16/fp32 bits exactly):
  q        [n_rows, H_q, d]   query rows of one request
  k_base   [H_kv, kv_len, d]  shared base cache (keys already rotated if the
                              model uses RoPE)
  v_base   [H_kv, kv_len, d]
  l_k, l_v [kv_len, r]        shared LR cache (never rotated as stored)
  b_k, b_v [r, H_kv * d]      one agent's up-projections
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "causal_visible",
    "rope_inv_freq",
    "rope_tables",
    "rope_rotate_half",
    "softmax_two_pass",
    "attention_materialised",
    "attention_reordered",
    "attention_augmented",
    "gather_pages",
    "decode_paged",
    "prefill",
    "lr_cache_build",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def causal_visible(q_pos, kv_len):
    """Boolean visibility ``[n_rows, kv_len]``: row at absolute position p sees keys 0..p.

    Reading (the pages are silent on alignment): new tokens are appended at the
    end of the accumulated context ``L = L_p + L_c`` (LRAgent App. B), so the
    i-th of ``q_len`` new tokens sits at position ``kv_len - q_len + i`` and
    attends to every earlier token and to itself.  A decode row sits at
    ``kv_len - 1`` and sees all keys.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(-1)
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    return j <= q_pos[:, None]


def rope_inv_freq(head_dim, theta):
    """Rotary frequencies ``theta^(-2i/d)`` for pair index ``i = 0 .. d/2-1``, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rope_tables(n_pos, head_dim, theta):
    """cos / sin of ``pos * theta^(-2i/d)``, shape ``[n_pos, d/2]``, float64."""
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * rope_inv_freq(head_dim, theta)[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate_half(x, cos, sin):
    """Rotate-half RoPE: pair ``(i, i + d/2)`` turned by the angle of row ``pos``.

    ``x`` is ``[n_pos, d]``; ``cos``/``sin`` are ``[n_pos, d/2]`` for the same rows.
    Reading: the pages name RoPE only (LRAgent App. D.1); the pairing used is the
    LLaMA convention of the model the pages evaluate.
    """
    x = _f64(x)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def softmax_two_pass(s):
    """Row softmax: subtract the row max of visible scores, exponentiate, normalise.

    Masked entries are ``-inf`` and come out as exact zeros.
    """
    s = _f64(s)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _check(q, k_base, v_base, l_k, l_v, b_k, b_v):
    n_rows, h_q, d = q.shape
    h_kv, kv_len, d2 = k_base.shape
    r = l_k.shape[1]
    assert d == d2 and v_base.shape == k_base.shape
    assert l_k.shape == (kv_len, r) and l_v.shape == (kv_len, r)
    assert b_k.shape == (r, h_kv * d) and b_v.shape == (r, h_kv * d)
    assert h_q % h_kv == 0
    return n_rows, h_q, h_kv, d, kv_len, r


def attention_materialised(q, k_base, v_base, l_k, l_v, b_k, b_v, *, q_pos=None,
                           rope=None, scale=None, row_chunk=1024, return_probs=False):
    """The definition: materialise the adapted K and V per KV head, then attend.

    For KV head ``h`` and the query heads ``hq`` with ``hq // (H_q/H_kv) == h``
    (grouped-query attention, contiguous groups):

      dK = L_k B_k[:, h-slice]             (App. A.3: dY = X A B, Y_lr = X A)
      dK = rot_pos(dK)  if rope is given   (App. D.1: rebuild before RoPE)
      K  = K_base[h] + dK
      V  = V_base[h] + L_v B_v[:, h-slice] (values are never rotated)
      S  = Q_hq K^T * scale,  scale = 1/sqrt(d) unless given
      S[i, j] = -inf where key j is after row i's position (bottom-right causal)
      P  = softmax(S) (two-pass), O_hq = P V

    ``q_pos`` holds each row's absolute position (default: all rows at
    ``kv_len - 1``, i.e. decode).  ``rope`` is ``(cos, sin)`` of shape
    ``[kv_len, d/2]`` indexed by absolute key position.  Rows are processed in
    chunks of ``row_chunk`` only to bound memory; every row is still the plain
    definition.  Returns ``O`` ``[n_rows, H_q, d]`` (and ``P`` per query head if
    ``return_probs``).
    """
    q, k_base, v_base, l_k, l_v, b_k, b_v = map(_f64, (q, k_base, v_base, l_k, l_v, b_k, b_v))
    n_rows, h_q, h_kv, d, kv_len, r = _check(q, k_base, v_base, l_k, l_v, b_k, b_v)
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.full(n_rows, kv_len - 1, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    assert q_pos.shape == (n_rows,) and np.all(q_pos < kv_len) and np.all(q_pos >= 0)
    out = np.empty((n_rows, h_q, d), dtype=np.float64)
    probs = np.empty((h_q, n_rows, kv_len)) if return_probs else None
    for h in range(h_kv):
        cols = slice(h * d, (h + 1) * d)
        dk = l_k @ b_k[:, cols]
        if rope is not None:
            cos, sin = rope
            dk = rope_rotate_half(dk, cos[:kv_len], sin[:kv_len])
        k_full = k_base[h] + dk
        v_full = v_base[h] + l_v @ b_v[:, cols]
        for hq in range(h * g, (h + 1) * g):
            for r0 in range(0, n_rows, row_chunk):
                r1 = min(n_rows, r0 + row_chunk)
                s = (q[r0:r1, hq, :] @ k_full.T) * scale
                s = np.where(causal_visible(q_pos[r0:r1], kv_len), s, -np.inf)
                p = softmax_two_pass(s)
                out[r0:r1, hq, :] = p @ v_full
                if return_probs:
                    probs[hq, r0:r1] = p
    return (out, probs) if return_probs else out


def attention_reordered(q, k_base, v_base, l_k, l_v, b_k, b_v, *, q_pos=None, scale=None):
    """Flash-LoRA reordering, written out without streaming (for pinning only).

    Score side:  ``Q K_base^T + (Q B_k^T) L_k^T`` — valid only without RoPE on
    the adapter key term (LRAgent App. D.1 says the rotation blocks this).
    Value side:  ``P V_base + (P V_lr) B_v`` (LRAgent §3, App. B: the
    attention-weighted sum is taken in rank r first and up-projected once).
    """
    q, k_base, v_base, l_k, l_v, b_k, b_v = map(_f64, (q, k_base, v_base, l_k, l_v, b_k, b_v))
    n_rows, h_q, h_kv, d, kv_len, r = _check(q, k_base, v_base, l_k, l_v, b_k, b_v)
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.full(n_rows, kv_len - 1, dtype=np.int64)
    vis = causal_visible(q_pos, kv_len)
    out = np.empty((n_rows, h_q, d))
    for hq in range(h_q):
        h = hq // g
        cols = slice(h * d, (h + 1) * d)
        qh = q[:, hq, :]
        s = (qh @ k_base[h].T + (qh @ b_k[:, cols].T) @ l_k.T) * scale
        p = softmax_two_pass(np.where(vis, s, -np.inf))
        out[:, hq, :] = p @ v_base[h] + (p @ l_v) @ b_v[:, cols]
    return out


def attention_augmented(q, k_base, v_base, l_k, l_v, b_k, b_v, *, q_pos=None, scale=None):
    """Augmented-head form of the reordering (for pinning only).

    ``q~ = [q, q B_k^T]``, ``k~_j = [k_base_j, l_k_j]``, ``v~_j = [v_base_j, l_v_j]``;
    ``O~ = softmax(q~ k~^T * scale) v~ = [O_base, O_lr]`` and ``O = O_base + O_lr B_v``.
    Same mathematics as ``attention_reordered`` with the two score terms fused
    into one product over ``d + r`` columns.
    """
    q, k_base, v_base, l_k, l_v, b_k, b_v = map(_f64, (q, k_base, v_base, l_k, l_v, b_k, b_v))
    n_rows, h_q, h_kv, d, kv_len, r = _check(q, k_base, v_base, l_k, l_v, b_k, b_v)
    g = h_q // h_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if q_pos is None:
        q_pos = np.full(n_rows, kv_len - 1, dtype=np.int64)
    vis = causal_visible(q_pos, kv_len)
    out = np.empty((n_rows, h_q, d))
    for hq in range(h_q):
        h = hq // g
        cols = slice(h * d, (h + 1) * d)
        q_aug = np.concatenate([q[:, hq, :], q[:, hq, :] @ b_k[:, cols].T], axis=1)
        k_aug = np.concatenate([k_base[h], l_k], axis=1)
        v_aug = np.concatenate([v_base[h], l_v], axis=1)
        p = softmax_two_pass(np.where(vis, (q_aug @ k_aug.T) * scale, -np.inf))
        o_aug = p @ v_aug
        out[:, hq, :] = o_aug[:, :d] + o_aug[:, d:] @ b_v[:, cols]
    return out


def gather_pages(kv_pool, l_pool, table_row, length):
    """Rebuild one context's contiguous caches from a paged pool.

    ``kv_pool`` is ``[n_pages, H_kv, page, d]`` and ``l_pool`` is
    ``[n_pages, page, r]``; logical token ``t`` lives in page
    ``table_row[t // page]`` at slot ``t % page`` (reading: paging is not on
    the pages; the LR pages share the base cache's block table).
    Returns ``([H_kv, length, d], [length, r])``.
    """
    n_pages, h_kv, page, d = kv_pool.shape
    r = l_pool.shape[2]
    kv = np.empty((h_kv, length, d), dtype=np.float64)
    lr = np.empty((length, r), dtype=np.float64)
    for blk in range((length + page - 1) // page):
        pid = int(table_row[blk])
        t0 = blk * page
        n = min(page, length - t0)
        kv[:, t0:t0 + n, :] = kv_pool[pid, :, :n, :]
        lr[t0:t0 + n, :] = l_pool[pid, :n, :]
    return kv, lr


def decode_paged(q, req_ctx, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table,
                 ctx_len, b_k, b_v, *, rope=None, scale=None, requests=None):
    """Decode: one new query token per request over its context's shared caches.

    ``q`` ``[n_req, H_q, d]``; request ``i`` reads context ``req_ctx[i]`` (its
    base and LR pages) with agent ``req_agent[i]``'s ``B_k``/``B_v``
    (``b_k``, ``b_v``: ``[n_agents, r, H_kv*d]``).  The newest token is part of
    the context, so the query sees all ``ctx_len[c]`` keys.  ``lk_pool`` /
    ``lv_pool`` are one LR pool shared by every agent (BaseLRShared, LRAgent §3)
    or, with a leading agent axis, one LR pool per agent (BaseShared: each agent
    keeps its own A and so its own LR cache); request ``i`` then reads agent
    ``req_agent[i]``'s pool through the same block table.  ``rope`` is
    ``(cos, sin)`` ``[>= max ctx_len, d/2]``: the adapter key term of the key at
    token index ``j`` of a context is rotated by row ``j`` (App. D.1, as in
    prefill).  ``requests`` optionally restricts which requests are evaluated
    (rows of the output for the others are left as NaN).
    """
    q = _f64(q)
    n_req, h_q, d = q.shape
    out = np.full((n_req, h_q, d), np.nan)
    idx = range(n_req) if requests is None else requests
    for i in idx:
        c, a = int(req_ctx[i]), int(req_agent[i])
        n = int(ctx_len[c])
        lkp = lk_pool[a] if np.ndim(lk_pool) == 4 else lk_pool
        lvp = lv_pool[a] if np.ndim(lv_pool) == 4 else lv_pool
        kb, lk = gather_pages(k_pool, lkp, block_table[c], n)
        vb, lv = gather_pages(v_pool, lvp, block_table[c], n)
        out[i] = attention_materialised(q[i][None], kb, vb, lk, lv, _f64(b_k[a]), _f64(b_v[a]),
                                        q_pos=[n - 1], rope=rope, scale=scale)[0]
    return out


def prefill(q, req_agent, k_base, v_base, l_k, l_v, b_k, b_v, *, rope=None, scale=None,
            rows=None, row_chunk=512):
    """Chunked prefill: each request's ``q_len`` new tokens over the shared context.

    ``q`` ``[n_req, q_len, H_q, d]``; the new tokens are the last ``q_len`` of
    the ``kv_len`` cached tokens (their base and LR rows are already in the
    caches), attended causally.  ``l_k`` / ``l_v`` are ``[kv_len, r]`` (shared)
    or ``[n_agents, kv_len, r]`` (one LR cache per agent, LRAgent §3
    BaseShared).  ``rows`` optionally selects the chunk-local query indices to
    evaluate (same for every request); the result then has ``len(rows)`` rows
    per request.
    """
    q = _f64(q)
    n_req, q_len, h_q, d = q.shape
    kv_len = k_base.shape[1]
    assert kv_len >= q_len
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((n_req, len(rows), h_q, d))
    for i in range(n_req):
        a = int(req_agent[i])
        lk = l_k[a] if np.ndim(l_k) == 3 else l_k
        lv = l_v[a] if np.ndim(l_v) == 3 else l_v
        out[i] = attention_materialised(q[i, rows], k_base, v_base, lk, lv,
                                        _f64(b_k[a]), _f64(b_v[a]),
                                        q_pos=kv_len - q_len + rows, rope=rope,
                                        scale=scale, row_chunk=row_chunk)
    return out


def lr_cache_build(x, a_k, a_v):
    """Shared low-rank cache rows for new tokens: ``L_k = X A_k``, ``L_v = X A_v``.

    PReCache (PreLRShared): an agent's LR cache is the hidden state times the
    adapter's input matrix, built when the context is first processed; under
    shared A (LRAgent §3 BaseLRShared) one product serves every agent.
    """
    x = _f64(x)
    return x @ _f64(a_k), x @ _f64(a_v)
