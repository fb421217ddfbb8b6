"""lra_attn_decode_noalloc (the decode entry point that allocates nothing) against
lra_attn_decode with a caller workspace: the same kernels read the library's own
scratch instead, so the rows must be identical, on consecutive calls that reuse the
scratch, the second one smaller."""
import os

import numpy as np
import pytest

import workloads as w
from gpu_helpers import DecodeDev, assert_parity, host, oracle_decode

pytestmark = pytest.mark.gpu


def _both(d, rope_theta=None):
    import torch
    import attention_shared_base_amd as lra
    cos = sin = None
    if rope_theta is not None:
        cos, sin = d.rope(rope_theta)
    ref = host(d.run(rope_theta=rope_theta))
    out = torch.full_like(d.q, float("nan"))
    lra.decode_noalloc(d.q, d.crs, d.agent, d.k, d.v, d.lk, d.lv, d.bt, d.clen, d.b_k, d.b_v, out,
                       max_req_per_ctx=d.max_req_per_ctx, max_ctx_len=d.max_ctx_len,
                       rope_cos=cos, rope_sin=sin)
    return host(out), ref


@pytest.mark.parametrize("persistent", ["0", "1"])
def test_noalloc_matches_workspace_decode_twice(persistent):
    big = w.make_decode(61, dtype="bf16", ctx_lens=[6000, 4096, 2500], reqs=[(0, 0), (0, 1), (0, 2),
                        (1, 1), (2, 2), (2, 0)], n_agents=3, h_q=32, h_kv=8, d=128, r=16,
                        shuffle=True, name="noalloc big")
    small = w.make_decode(62, dtype="bf16", ctx_lens=[1500, 700], reqs=[(0, 1), (1, 0)], n_agents=2,
                          h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="noalloc small")
    try:
        os.environ["LRA_DECODE_CHUNK"] = "512"
        os.environ["LRA_DECODE_PERSISTENT"] = persistent
        for case in (big, small):
            d = DecodeDev(case)
            got, ref = _both(d)
            print(f"[noalloc] {case.name} persistent={persistent}: equal={np.array_equal(got, ref)}",
                  flush=True)
            assert np.array_equal(got, ref), f"{case.name}: differs from the workspace decode"
            assert_parity(got, oracle_decode(case), "bf16", case.name)
    finally:
        os.environ.pop("LRA_DECODE_CHUNK", None)
        os.environ.pop("LRA_DECODE_PERSISTENT", None)


def test_noalloc_primary_shape_and_rope():
    """The primary decode shape (4 x 8192-token contexts, 16 requests), then a smaller
    RoPE call on the same scratch."""
    d = DecodeDev(w.config2())
    got, ref = _both(d)
    assert np.array_equal(got, ref)
    case = w.make_decode(63, dtype="bf16", ctx_lens=[3000, 1200], reqs=[(0, 0), (0, 1), (1, 1)],
                         n_agents=2, h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="noalloc rope")
    d = DecodeDev(case)
    got, ref = _both(d, rope_theta=500000.0)
    assert np.array_equal(got, ref)
