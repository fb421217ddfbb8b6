"""Shared helpers of the GPU parity tests: upload seeded inputs, call the HIP path
through the C-ABI binding, widen results, compare with the oracle."""
from __future__ import annotations

import numpy as np

import workloads as w

# Parity bars.  fp32: max-abs 1e-5.  bf16 storage / fp32 accumulation:
# max-abs 2e-2 and relative L2 1e-2; the adapter's own contribution
# (O - O with B = 0) must match the oracle's to relative L2 5e-2 so that a
# dropped or garbled low-rank path cannot hide under the base attention.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
DELTA_REL_L2 = 5e-2


def dev(a):
    """numpy storage array -> torch tensor on cuda:0 (uint16 = bf16 bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to("cuda")
    if a.dtype in (np.int32, np.int64):
        return torch.from_numpy(a.astype(np.int32)).to("cuda")
    raise TypeError(a.dtype)


def host(t):
    """torch device tensor -> float64 numpy (exact widening of bf16/fp32)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)) if err.size else 0.0
    return max_abs, rel


def assert_parity(got, ref, dtype, what=""):
    max_abs, rel = metrics(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, \
            f"{what}: max-abs {max_abs:.3e} (bar {BF16_MAX_ABS}), rel-L2 {rel:.3e} (bar {BF16_REL_L2})"
    return max_abs, rel


# ------------------------------------------------------------------ decode

class DecodeDev:
    """A DecodeCase uploaded in the kernel's page layouts."""

    def __init__(self, case: w.DecodeCase):
        self.case = case
        k, v, lk, lv = w.decode_device_layout(case.k_pool, case.v_pool, case.lk_pool, case.lv_pool)
        self.q = dev(case.q)
        self.k, self.v, self.lk, self.lv = dev(k), dev(v), dev(lk), dev(lv)
        self.crs = dev(case.ctx_req_start())
        self.agent = dev(case.req_agent)
        self.bt = dev(case.block_table)
        self.clen = dev(case.ctx_len)
        self.b_k, self.b_v = dev(case.b_k), dev(case.b_v)
        counts = np.bincount(case.req_ctx, minlength=case.n_ctx)
        self.max_req_per_ctx = int(max(1, counts.max()))
        self.max_ctx_len = int(case.ctx_len.max())
        self._rope = {}

    def rope(self, theta):
        """fp32 RoPE tables [max(max_ctx_len, 1), d/2] built on the GPU (cached per theta)."""
        import attention_shared_base_amd as lra
        if theta not in self._rope:
            self._rope[theta] = lra.rope_table(theta, self.case.d, max(self.max_ctx_len, 1))
        return self._rope[theta]

    def run(self, out=None, workspace=None, b_k=None, b_v=None, q=None, rope_theta=None, lk=None,
            lv=None):
        import attention_shared_base_amd as lra
        cos = sin = None
        if rope_theta is not None:
            cos, sin = self.rope(rope_theta)
        return lra.decode(self.q if q is None else q, self.crs, self.agent, self.k, self.v,
                          self.lk if lk is None else lk, self.lv if lv is None else lv,
                          self.bt, self.clen,
                          self.b_k if b_k is None else b_k, self.b_v if b_v is None else b_v,
                          max_req_per_ctx=self.max_req_per_ctx, max_ctx_len=self.max_ctx_len,
                          rope_cos=cos, rope_sin=sin, out=out, workspace=workspace)


def oracle_decode(case: w.DecodeCase, requests=None, zero_b=False, rope_theta=None):
    import oracle
    bk = np.zeros_like(w.widen(case.b_k)) if zero_b else w.widen(case.b_k)
    bv = np.zeros_like(w.widen(case.b_v)) if zero_b else w.widen(case.b_v)
    rope = None
    if rope_theta is not None:
        rope = oracle.rope_tables(max(int(case.ctx_len.max()), 1), case.d, rope_theta)
    return oracle.decode_paged(w.widen(case.q), case.req_ctx, case.req_agent,
                               w.widen(case.k_pool), w.widen(case.v_pool), w.widen(case.lk_pool),
                               w.widen(case.lv_pool), case.block_table, case.ctx_len, bk, bv,
                               rope=rope, requests=requests)


# ------------------------------------------------------------------ prefill

class PrefillDev:
    def __init__(self, case: w.PrefillCase, rope=True):
        import attention_shared_base_amd as lra
        self.case = case
        self.q = dev(case.q)
        self.agent = dev(case.req_agent)
        self.k, self.v = dev(case.k_base), dev(case.v_base)
        self.lk, self.lv = dev(case.l_k), dev(case.l_v)
        self.b_k, self.b_v = dev(case.b_k), dev(case.b_v)
        self.cos = self.sin = None
        if rope and case.rope_theta is not None:
            self.cos, self.sin = lra.rope_table(case.rope_theta, case.d, case.kv_len)

    def run(self, out=None, b_k=None, b_v=None, lk=None, lv=None):
        import attention_shared_base_amd as lra
        return lra.prefill(self.q, self.agent, self.k, self.v,
                           self.lk if lk is None else lk, self.lv if lv is None else lv,
                           self.b_k if b_k is None else b_k, self.b_v if b_v is None else b_v,
                           rope_cos=self.cos, rope_sin=self.sin, out=out)


def oracle_prefill(case: w.PrefillCase, rows=None, zero_b=False, l_k=None, l_v=None,
                   requests=None):
    import oracle
    rope = (oracle.rope_tables(case.kv_len, case.d, case.rope_theta)
            if case.rope_theta is not None else None)
    bk = np.zeros_like(w.widen(case.b_k)) if zero_b else w.widen(case.b_k)
    bv = np.zeros_like(w.widen(case.b_v)) if zero_b else w.widen(case.b_v)
    q = w.widen(case.q)
    agents = case.req_agent
    if requests is not None:
        q = q[requests]
        agents = agents[requests]
    return oracle.prefill(q, agents, w.widen(case.k_base), w.widen(case.v_base),
                          w.widen(case.l_k) if l_k is None else l_k,
                          w.widen(case.l_v) if l_v is None else l_v, bk, bv, rope=rope,
                          rows=rows)
