"""The five synthetic workloads (LLaMA-3.1-8B attention shapes) and generic builders.

The pages evaluate LLaMA-3.1-8B-Instruct / Ministral-8B-Instruct on HotpotQA and
ScienceQA agent trajectories (LRAgent §4, App. C.6: retrieved context 0.25k-16k,
total trajectory 1.9k-66.4k tokens).  Neither models, adapters nor traces are
available here, so seeded N(0, sigma^2) tensors with those shapes stand in:

1. tiny fp32 decode + prefill: 1 context of 256 tokens (240 old + 16 new),
   2 agents, H_q 4, H_kv 2, d 64, r 8, B ~ N(0, 0.1^2);
2. bf16 decode: 4 shared contexts x 8192 tokens, 16 requests (request b on
   context b // 4 with agent b % 4), H_q 32, H_kv 8, d 128, r 16,
   B ~ N(0, 0.05^2);
3. bf16 chunked prefill with RoPE (theta 500000) on the adapter key term:
   512 new tokens over 16384 old ones (kv 16896), 4 agents, r 16;
4. bf16 paged decode: 32 contexts with lengths uniform in [4096, 65536],
   16-token pages placed by a random permutation of the pool, 32 requests
   (request b on context b with agent b % 8), r 32;
5. bf16 PreLRShared step per layer: X [4096, 4096], A_k, A_v [4096, 16] ~
   N(0, 1/4096), base cache of 135168 tokens (131072 old + 4096 new), LR rows
   of the old tokens ~ N(0, 1), 8 agents each prefilling the 4096 new tokens.

Everything not stated above is N(0, 1).  Storage is bf16 bits (uint16) or
float32; see ``workloads.synth`` for the stream recipe.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .synth import (TAG_AK, TAG_AV, TAG_BK, TAG_BV, TAG_K, TAG_LEN, TAG_LK, TAG_LV,
                    TAG_PERM, TAG_Q, TAG_QDEC, TAG_V, TAG_X, draw, paginate, rng_for)

PAGE = 16


@dataclass
class DecodeCase:
    """Inputs of one paged decode call.  Requests are grouped by context."""
    dtype: str
    h_q: int
    h_kv: int
    d: int
    r: int
    page: int
    q: np.ndarray            # [n_req, H_q, d]
    req_ctx: np.ndarray      # [n_req] int32, non-decreasing
    req_agent: np.ndarray    # [n_req] int32
    ctx_len: np.ndarray      # [n_ctx] int32
    block_table: np.ndarray  # [n_ctx, max_blocks] int32
    k_pool: np.ndarray       # [n_pages, H_kv, page, d]
    v_pool: np.ndarray
    lk_pool: np.ndarray      # [n_pages, page, r]
    lv_pool: np.ndarray
    b_k: np.ndarray          # [n_agents, r, H_kv*d]
    b_v: np.ndarray
    name: str = ""

    @property
    def n_req(self):
        return self.q.shape[0]

    @property
    def n_ctx(self):
        return self.ctx_len.shape[0]

    @property
    def n_agents(self):
        return self.b_k.shape[0]

    def ctx_req_start(self):
        """CSR offsets: requests of context c are ``start[c] .. start[c+1]-1``."""
        start = np.zeros(self.n_ctx + 1, dtype=np.int32)
        np.add.at(start, self.req_ctx.astype(np.int64) + 1, 1)
        return np.cumsum(start).astype(np.int32)


@dataclass
class PrefillCase:
    """Inputs of one chunked-prefill call over one shared context."""
    dtype: str
    h_q: int
    h_kv: int
    d: int
    r: int
    q: np.ndarray          # [n_req, q_len, H_q, d]
    req_agent: np.ndarray  # [n_req] int32
    k_base: np.ndarray     # [H_kv, kv_len, d]
    v_base: np.ndarray
    l_k: np.ndarray        # [kv_len, r]
    l_v: np.ndarray
    b_k: np.ndarray        # [n_agents, r, H_kv*d]
    b_v: np.ndarray
    rope_theta: Optional[float] = None
    name: str = ""

    @property
    def n_req(self):
        return self.q.shape[0]

    @property
    def q_len(self):
        return self.q.shape[1]

    @property
    def kv_len(self):
        return self.k_base.shape[1]


@dataclass
class LRBuildCase:
    dtype: str
    x: np.ndarray    # [n_tok, d_model]
    a_k: np.ndarray  # [r, d_model]  (LoRA A weight layout, out x in: L = X a_k^T)
    a_v: np.ndarray
    name: str = ""


@dataclass
class PreLRLayerCase:
    """One layer of the PreLRShared step: LR build of the new rows, then prefill."""
    lr: LRBuildCase
    prefill: PrefillCase          # l_k / l_v hold the OLD rows only (prefix)
    n_old: int
    extra: dict = field(default_factory=dict)


# ----------------------------------------------------------------------------------
# generic builders


def page_table(seed, ctx_lens, *, shuffle, page=PAGE, max_blocks=None, layer=0):
    """Block table ``[n_ctx, max_blocks]`` over a pool of exactly sum(ceil(len/page)) pages.

    Contexts take consecutive pool pages in order, or (``shuffle``) the pages of a
    random permutation of the pool.  Unused table entries are 0.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    n_ctx = len(ctx_lens)
    nblk = (ctx_lens + page - 1) // page
    n_pages = int(max(1, nblk.sum()))
    if max_blocks is None:
        max_blocks = int(max(1, nblk.max()))
    order = (rng_for(seed, TAG_PERM, layer).permutation(n_pages) if shuffle
             else np.arange(n_pages))
    table = np.zeros((n_ctx, max_blocks), dtype=np.int32)
    off = 0
    for c in range(n_ctx):
        table[c, :nblk[c]] = order[off:off + nblk[c]]
        off += int(nblk[c])
    return table, n_pages


def make_decode(seed, *, dtype, ctx_lens, reqs, n_agents, h_q, h_kv, d, r, page=PAGE,
                shuffle=False, q_sigma=1.0, b_sigma=0.05, kv_sigma=1.0, l_sigma=1.0,
                max_blocks=None, name="", layer=0):
    """Paged decode inputs.  ``reqs`` is a list of ``(ctx, agent)`` sorted by ctx."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    table, n_pages = page_table(seed, ctx_lens, shuffle=shuffle, page=page,
                                max_blocks=max_blocks, layer=layer)
    req_ctx = np.array([c for c, _ in reqs], dtype=np.int32)
    req_agent = np.array([a for _, a in reqs], dtype=np.int32)
    assert np.all(np.diff(req_ctx) >= 0), "requests must be grouped by context"
    return DecodeCase(
        dtype=dtype, h_q=h_q, h_kv=h_kv, d=d, r=r, page=page,
        q=draw(seed, TAG_QDEC, (len(reqs), h_q, d), q_sigma, dtype, layer),
        req_ctx=req_ctx, req_agent=req_agent,
        ctx_len=ctx_lens.astype(np.int32), block_table=table,
        k_pool=draw(seed, TAG_K, (n_pages, h_kv, page, d), kv_sigma, dtype, layer),
        v_pool=draw(seed, TAG_V, (n_pages, h_kv, page, d), kv_sigma, dtype, layer),
        lk_pool=draw(seed, TAG_LK, (n_pages, page, r), l_sigma, dtype, layer),
        lv_pool=draw(seed, TAG_LV, (n_pages, page, r), l_sigma, dtype, layer),
        b_k=draw(seed, TAG_BK, (n_agents, r, h_kv * d), b_sigma, dtype, layer),
        b_v=draw(seed, TAG_BV, (n_agents, r, h_kv * d), b_sigma, dtype, layer),
        name=name)


def decode_subset(case: DecodeCase, requests) -> DecodeCase:
    """The same decode restricted to ``requests``: their contexts and only those
    contexts' pages, copied into a compact pool with the block tables renumbered.
    Pure data movement (every kept value is bit-identical), so that a reference can
    widen a few requests' caches instead of the whole pool.  The kept requests come
    in ascending order (requests are grouped by context, so this is context order)."""
    requests = sorted({int(i) for i in requests})
    ctxs = sorted({int(case.req_ctx[i]) for i in requests})
    new_ctx = {c: j for j, c in enumerate(ctxs)}
    page = case.page
    nblk = [(int(case.ctx_len[c]) + page - 1) // page for c in ctxs]
    max_blocks = max(1, max(nblk))
    old_ids = np.concatenate([case.block_table[c, :n] for c, n in zip(ctxs, nblk)] + [np.zeros(0, np.int32)])
    table = np.zeros((len(ctxs), max_blocks), dtype=np.int32)
    off = 0
    for j, n in enumerate(nblk):
        table[j, :n] = np.arange(off, off + n)
        off += n
    ids = old_ids if off > 0 else np.zeros(1, np.int64)
    reqs = requests
    return DecodeCase(
        dtype=case.dtype, h_q=case.h_q, h_kv=case.h_kv, d=case.d, r=case.r, page=page,
        q=case.q[reqs], req_ctx=np.array([new_ctx[int(case.req_ctx[i])] for i in reqs], np.int32),
        req_agent=case.req_agent[reqs], ctx_len=case.ctx_len[ctxs].astype(np.int32),
        block_table=table, k_pool=case.k_pool[ids], v_pool=case.v_pool[ids],
        lk_pool=case.lk_pool[ids], lv_pool=case.lv_pool[ids], b_k=case.b_k, b_v=case.b_v,
        name=f"{case.name} (requests {reqs})")


def make_prefill(seed, *, dtype, kv_len, q_len, req_agents, n_agents, h_q, h_kv, d, r,
                 rope_theta=None, q_sigma=1.0, b_sigma=0.05, name="", layer=0):
    n_req = len(req_agents)
    return PrefillCase(
        dtype=dtype, h_q=h_q, h_kv=h_kv, d=d, r=r,
        q=draw(seed, TAG_Q, (n_req, q_len, h_q, d), q_sigma, dtype, layer),
        req_agent=np.asarray(req_agents, dtype=np.int32),
        k_base=draw(seed, TAG_K, (h_kv, kv_len, d), 1.0, dtype, layer),
        v_base=draw(seed, TAG_V, (h_kv, kv_len, d), 1.0, dtype, layer),
        l_k=draw(seed, TAG_LK, (kv_len, r), 1.0, dtype, layer),
        l_v=draw(seed, TAG_LV, (kv_len, r), 1.0, dtype, layer),
        b_k=draw(seed, TAG_BK, (n_agents, r, h_kv * d), b_sigma, dtype, layer),
        b_v=draw(seed, TAG_BV, (n_agents, r, h_kv * d), b_sigma, dtype, layer),
        rope_theta=rope_theta, name=name)


def make_lr_build(seed, *, dtype, n_tok, d_model, r, a_sigma=None, name="", layer=0):
    if a_sigma is None:
        a_sigma = 1.0 / np.sqrt(d_model)
    return LRBuildCase(
        dtype=dtype,
        x=draw(seed, TAG_X, (n_tok, d_model), 1.0, dtype, layer),
        a_k=draw(seed, TAG_AK, (r, d_model), a_sigma, dtype, layer),
        a_v=draw(seed, TAG_AV, (r, d_model), a_sigma, dtype, layer),
        name=name)


# ----------------------------------------------------------------------------------
# the five workloads


def config1():
    """Tiny fp32 case: returns ``(DecodeCase, PrefillCase)`` over the same caches."""
    seed, dt = 1, "f32"
    h_q, h_kv, d, r, kv_len, q_len = 4, 2, 64, 8, 256, 16
    pre = make_prefill(seed, dtype=dt, kv_len=kv_len, q_len=q_len, req_agents=[0, 1],
                       n_agents=2, h_q=h_q, h_kv=h_kv, d=d, r=r, b_sigma=0.1,
                       name="cfg1-prefill: fp32 kv256 (240+16) 2 agents Hq4 Hkv2 d64 r8")
    n_pages = kv_len // PAGE
    ids = np.arange(n_pages)
    kp, lkp = paginate(pre.k_base, pre.l_k, ids, n_pages, PAGE)
    vp, lvp = paginate(pre.v_base, pre.l_v, ids, n_pages, PAGE)
    dec = DecodeCase(
        dtype=dt, h_q=h_q, h_kv=h_kv, d=d, r=r, page=PAGE,
        q=draw(seed, TAG_QDEC, (2, h_q, d), 1.0, dt),
        req_ctx=np.array([0, 0], np.int32), req_agent=np.array([0, 1], np.int32),
        ctx_len=np.array([kv_len], np.int32), block_table=ids.astype(np.int32)[None, :],
        k_pool=kp, v_pool=vp, lk_pool=lkp, lv_pool=lvp, b_k=pre.b_k, b_v=pre.b_v,
        name="cfg1-decode: fp32 kv256 2 agents Hq4 Hkv2 d64 r8")
    return dec, pre


def config2(seed=2, layer=0):
    reqs = [(b // 4, b % 4) for b in range(16)]
    return make_decode(seed, dtype="bf16", ctx_lens=[8192] * 4, reqs=reqs, n_agents=4,
                       h_q=32, h_kv=8, d=128, r=16, shuffle=False, layer=layer,
                       name="cfg2-decode: bf16 4 ctx x 8192, 16 req (4 agents/ctx), "
                            "Hq32 Hkv8 d128 r16")


def config3(seed=3, layer=0):
    return make_prefill(seed, dtype="bf16", kv_len=16384 + 512, q_len=512,
                        req_agents=[0, 1, 2, 3], n_agents=4, h_q=32, h_kv=8, d=128, r=16,
                        rope_theta=500000.0, layer=layer,
                        name="cfg3-prefill: bf16 512 new over 16384, 4 agents, RoPE 5e5, "
                             "Hq32 Hkv8 d128 r16")


def config4_lengths(seed=4, layer=0):
    return rng_for(seed, TAG_LEN, layer).integers(4096, 65536, size=32, endpoint=True)


def config4(seed=4, layer=0):
    lens = config4_lengths(seed, layer)
    reqs = [(b, b % 8) for b in range(32)]
    return make_decode(seed, dtype="bf16", ctx_lens=lens, reqs=reqs, n_agents=8,
                       h_q=32, h_kv=8, d=128, r=32, shuffle=True, max_blocks=65536 // PAGE,
                       layer=layer,
                       name="cfg4-paged-decode: bf16 32 ctx, len U[4096,65536], shuffled "
                            "16-tok pages, 8 agents, Hq32 Hkv8 d128 r32")


def config5_layer(layer, seed=5, n_new=4096, n_old=131072, d_model=4096, n_agents=8):
    """One layer of the PreLRShared step (sizes overridable for scaled-down tests)."""
    dt, h_q, h_kv, d, r = "bf16", 32, 8, 128, 16
    kv_len = n_old + n_new
    lr = make_lr_build(seed, dtype=dt, n_tok=n_new, d_model=d_model, r=r, layer=layer,
                       name=f"cfg5-lrbuild layer {layer}")
    pre = PrefillCase(
        dtype=dt, h_q=h_q, h_kv=h_kv, d=d, r=r,
        q=draw(seed, TAG_Q, (n_agents, n_new, h_q, d), 1.0, dt, layer),
        req_agent=np.arange(n_agents, dtype=np.int32),
        k_base=draw(seed, TAG_K, (h_kv, kv_len, d), 1.0, dt, layer),
        v_base=draw(seed, TAG_V, (h_kv, kv_len, d), 1.0, dt, layer),
        l_k=draw(seed, TAG_LK, (n_old, r), 1.0, dt, layer),
        l_v=draw(seed, TAG_LV, (n_old, r), 1.0, dt, layer),
        b_k=draw(seed, TAG_BK, (n_agents, r, h_kv * d), 0.05, dt, layer),
        b_v=draw(seed, TAG_BV, (n_agents, r, h_kv * d), 0.05, dt, layer),
        rope_theta=None, name=f"cfg5-prefill layer {layer}: {n_new} new over {n_old}")
    return PreLRLayerCase(lr=lr, prefill=pre, n_old=n_old)
