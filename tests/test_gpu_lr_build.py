"""GPU parity of the LR-cache build (lra_lr_cache_build) and the RoPE tables."""
import numpy as np
import pytest

import oracle
import workloads as w
from gpu_helpers import dev, host, metrics

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_tok,d_model,r,dtype,offset", [
    (100, 512, 16, "bf16", 0),
    (33, 256, 8, "bf16", 7),
    (64, 1024, 32, "bf16", 100),
    (4096, 4096, 16, "bf16", 131072),   # one layer of the 4096-new-token PreLRShared step
    (17, 96, 16, "f32", 3),
    (40, 4096, 32, "f32", 0),
])
def test_lr_build(n_tok, d_model, r, dtype, offset):
    import torch
    import attention_shared_base_amd as lra
    case = w.make_lr_build(41, dtype=dtype, n_tok=n_tok, d_model=d_model, r=r)
    x, ak, av = dev(case.x), dev(case.a_k), dev(case.a_v)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = offset + n_tok + 5
    lk = torch.full((rows, r), 7.0, dtype=tdt, device="cuda")
    lv = torch.full((rows, r), 7.0, dtype=tdt, device="cuda")
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
