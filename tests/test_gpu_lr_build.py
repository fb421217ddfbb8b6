"""GPU parity of the LR-cache build (lra_lr_cache_build) and the RoPE tables.

lra_lr_cache_build runs one of three kernels: the LDS-staged one (the default when d_model
is a multiple of its stage), the d_model-split one (workspace given) and the single-pass
one; LRA_LR_BUILD_PATH = split | single selects the latter two, so each is tested."""
import contextlib
import os

import numpy as np
import pytest

import oracle
import workloads as w
from gpu_helpers import dev, host, metrics

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def lr_path(name):
    """Run the LR builds of the block on kernel `name` (lds = the default choice)."""
    old = os.environ.pop("LRA_LR_BUILD_PATH", None)
    if name != "lds":
        os.environ["LRA_LR_BUILD_PATH"] = name
    try:
        yield
    finally:
        os.environ.pop("LRA_LR_BUILD_PATH", None)
        if old is not None:
            os.environ["LRA_LR_BUILD_PATH"] = old


@pytest.mark.parametrize("n_tok,d_model,r,dtype,offset", [
    (100, 512, 16, "bf16", 0),
    (33, 256, 8, "bf16", 7),
    (64, 1024, 32, "bf16", 100),
    (4096, 4096, 16, "bf16", 131072),   # one layer of the 4096-new-token PreLRShared step
    (17, 96, 16, "f32", 3),
    (40, 4096, 32, "f32", 0),
    (64, 512, 4, "bf16", 3),
    (23, 256, 4, "f32", 1),
])
@pytest.mark.parametrize("path", ["lds", "single"])
def test_lr_build(n_tok, d_model, r, dtype, offset, path):
    import torch
    import attention_shared_base_amd as lra
    case = w.make_lr_build(41, dtype=dtype, n_tok=n_tok, d_model=d_model, r=r)
    x, ak, av = dev(case.x), dev(case.a_k), dev(case.a_v)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = offset + n_tok + 5
    lk = torch.full((rows, r), 7.0, dtype=tdt, device="cuda")
    lv = torch.full((rows, r), 7.0, dtype=tdt, device="cuda")
    with lr_path(path):
        lra.lr_cache_build(x, ak, av, lk, lv, row_offset=offset)
    ref_k, ref_v = oracle.lr_cache_build(w.widen(case.x), w.widen(case.a_k).T, w.widen(case.a_v).T)
    gk, gv = host(lk), host(lv)
    assert np.all(gk[:offset] == 7.0) and np.all(gk[offset + n_tok:] == 7.0)
    assert np.all(gv[:offset] == 7.0) and np.all(gv[offset + n_tok:] == 7.0)
    for got, ref in ((gk[offset:offset + n_tok], ref_k), (gv[offset:offset + n_tok], ref_v)):
        ma, rel = metrics(got, ref)
        print(f"[lr-build] {n_tok}x{d_model} r{r} {dtype}: max-abs {ma:.2e} rel-L2 {rel:.2e}")
        if dtype == "f32":
            assert ma <= 1e-5 * max(1.0, np.max(np.abs(ref))) * np.sqrt(d_model / 64)
        else:
            # one bf16 rounding of the fp32-accumulated result
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3)
            assert rel <= 4e-3


def test_rope_tables_match_oracle():
    import attention_shared_base_amd as lra
    cos, sin = lra.rope_table(500000.0, 128, 16896)
    rc, rs = oracle.rope_tables(16896, 128, 500000.0)
    assert np.max(np.abs(host(cos) - rc)) < 1e-6
    assert np.max(np.abs(host(sin) - rs)) < 1e-6


@pytest.mark.parametrize("n_tok,d_model,r,n_lr", [
    (4096, 4096, 16, 1),    # 64 token blocks x 4 ranges of d_model
    (1000, 4096, 32, 1),    # ragged last block, 8 ranges
    (77, 1024, 8, 3),       # three agents, 2 ranges
    (20000, 2048, 16, 1),   # no split (enough blocks): the 64-token kernel alone
    (1000, 4096, 4, 2),     # rank 4: half of one 16-column tile
])
def test_lr_build_split_matches_oracle_and_single_pass(n_tok, d_model, r, n_lr):
    """The d_model-split build (workspace given) against the oracle within one bf16 rounding,
    against the single-pass build (no workspace) within two roundings, repeatable bit for
    bit, and leaving the workspace zeroed."""
    import torch
    import attention_shared_base_amd as lra
    rng = np.random.default_rng(43)
    x = w.f32_to_bf16_bits(rng.standard_normal((n_tok, d_model)).astype(np.float32))
    shp = (n_lr, r, d_model) if n_lr > 1 else (r, d_model)
    a_k = w.f32_to_bf16_bits((rng.standard_normal(shp) / 64).astype(np.float32))
    a_v = w.f32_to_bf16_bits((rng.standard_normal(shp) / 64).astype(np.float32))
    off = 5
    rows = off + n_tok + 3
    lshape = (n_lr, rows, r) if n_lr > 1 else (rows, r)
    n_ws = lra.lr_cache_build_workspace_size(dtype=1, n_tok=n_tok, d_model=d_model, rank=r, n_lr=n_lr)
    ws = torch.zeros(max(n_ws, 16), dtype=torch.uint8, device="cuda")
    outs = []
    for split in (True, True, False):
        lk = torch.full(lshape, 7.0, dtype=torch.bfloat16, device="cuda")
        lv = torch.full(lshape, 7.0, dtype=torch.bfloat16, device="cuda")
        with lr_path("split" if split else "single"):
            lra.lr_cache_build(dev(x), dev(a_k), dev(a_v), lk, lv, row_offset=off,
                               workspace=ws if split else None, split=split)
        outs.append((host(lk).reshape(n_lr, rows, r), host(lv).reshape(n_lr, rows, r)))
    units = -(-n_tok // 64) * n_lr
    assert int(ws[:4 * units].view(torch.int32).abs().sum()) == 0  # counters back at zero
    (sk, sv), (sk2, sv2), (pk, pv) = outs
    assert np.array_equal(sk, sk2) and np.array_equal(sv, sv2)
    ak3 = a_k.reshape(n_lr, r, d_model)
    av3 = a_v.reshape(n_lr, r, d_model)
    for a in range(n_lr):
        ek, ev = oracle.lr_cache_build(w.widen(x), w.widen(ak3[a]).T, w.widen(av3[a]).T)
        for got, single, e in ((sk[a], pk[a], ek), (sv[a], pv[a], ev)):
            assert np.all(got[:off] == 7.0) and np.all(got[off + n_tok:] == 7.0)
            g = got[off:off + n_tok]
            # fp32 accumulation in another order, one bf16 rounding
            assert np.all(np.abs(g - e) <= 2.0 ** -8 * np.abs(e) + 1e-3)
            assert np.all(np.abs(g - single[off:off + n_tok]) <= 2.0 ** -7 * np.abs(e) + 2e-3)


@pytest.mark.parametrize("n_tok,d_model,r,n_lr", [
    (4096, 4096, 16, 1),    # the PreLRShared layer: 256 workgroups, 16 stages
    (1000, 4096, 32, 1),    # ragged last block (8 tokens), rank 32: 3-stage ring
    (77, 1024, 8, 3),       # three agents, rank 8: 512-wide stages
    (16, 4096, 16, 1),      # one decode step's new rows: one workgroup
    (1000, 4096, 4, 2),     # rank 4: half of one 16-column tile
    (33, 256, 16, 1),       # a single stage
    (300, 768, 16, 2),      # stages fewer than the ring
])
def test_lr_build_lds_kernel(n_tok, d_model, r, n_lr):
    """The LDS-staged build: within one bf16 rounding of the oracle, within two of the split
    build, repeatable bit for bit, rows outside [row_offset, row_offset + n_tok) untouched,
    and n agents in one call give the bits of n single-agent calls."""
    import torch
    import attention_shared_base_amd as lra
    rng = np.random.default_rng(44)
    x = w.f32_to_bf16_bits(rng.standard_normal((n_tok, d_model)).astype(np.float32))
    a_k = w.f32_to_bf16_bits((rng.standard_normal((n_lr, r, d_model)) / 64).astype(np.float32))
    a_v = w.f32_to_bf16_bits((rng.standard_normal((n_lr, r, d_model)) / 64).astype(np.float32))
    off, rows = 5, 5 + n_tok + 3

    def build(path, ak, av, n):
        lk = torch.full((n, rows, r), 7.0, dtype=torch.bfloat16, device="cuda")
        lv = torch.full((n, rows, r), 7.0, dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(16, lra.lr_cache_build_workspace_size(dtype=1, n_tok=n_tok, d_model=d_model,
                                                                   rank=r, n_lr=n)), dtype=torch.uint8,
                         device="cuda")
        sq = n == 1
        with lr_path(path):
            lra.lr_cache_build(dev(x), dev(ak[0] if sq else ak), dev(av[0] if sq else av),
                               lk[0] if sq else lk, lv[0] if sq else lv, row_offset=off, workspace=ws)
        return host(lk), host(lv)

    lds1, lds2, split = build("lds", a_k, a_v, n_lr), build("lds", a_k, a_v, n_lr), build("split", a_k, a_v, n_lr)
    assert all(np.array_equal(u, v) for u, v in zip(lds1, lds2))
    for a in range(n_lr):
        ek, ev = oracle.lr_cache_build(w.widen(x), w.widen(a_k[a]).T, w.widen(a_v[a]).T)
        one = build("lds", a_k[a:a + 1], a_v[a:a + 1], 1)
        for got, sp, single, e in ((lds1[0][a], split[0][a], one[0][0], ek), (lds1[1][a], split[1][a], one[1][0], ev)):
            assert np.all(got[:off] == 7.0) and np.all(got[off + n_tok:] == 7.0)
            g = got[off:off + n_tok]
            assert np.all(np.abs(g - e) <= 2.0 ** -8 * np.abs(e) + 1e-3)
            assert np.all(np.abs(g - sp[off:off + n_tok]) <= 2.0 ** -7 * np.abs(e) + 2e-3)
            assert np.array_equal(got, single)
        ma, rel = metrics(lds1[0][a][off:off + n_tok], ek)
        print(f"[lr-build lds] {n_tok}x{d_model} r{r} agent {a}: max-abs {ma:.2e} rel-L2 {rel:.2e}", flush=True)
