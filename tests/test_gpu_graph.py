"""HIP-graph capture and stream concurrency of the hot path.  An LR-cache build (split over
d_model, workspace in use), a RoPE prefill and a split-K decode are recorded once in a torch CUDA
graph, then replayed with new inputs copied in eagerly between replays: every replay equals the
eager calls on the same inputs bit for bit, and eager calls between replays still do (the kernels
take fixed buffers, reset their own workspace counters and add no memset nodes).  Two decode
streams with their own workspaces running at once equal the same calls run in turn."""
import numpy as np
import pytest

import workloads as w
from gpu_helpers import DecodeDev, PrefillDev, dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    import torch
    import attention_shared_base_amd as lra
    dcase = w.make_decode(91, dtype="bf16", ctx_lens=[3000, 700], reqs=[(0, 0), (0, 1), (1, 1)],
                          n_agents=2, h_q=32, h_kv=8, d=128, r=16, shuffle=True, name="graph decode")
    dd = DecodeDev(dcase)
    d_ws = torch.zeros(lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1, n_req=3, n_ctx=2,
        max_req_per_ctx=dd.max_req_per_ctx, max_ctx_len=dd.max_ctx_len), dtype=torch.uint8,
        device="cuda")
    assert d_ws.numel() > 0  # several chunks per unit: the split-K merge runs
    d_out = torch.empty_like(dd.q)
    pcase = w.make_prefill(92, dtype="bf16", kv_len=600, q_len=64, req_agents=[1, 0], n_agents=2,
                           h_q=32, h_kv=8, d=128, r=16, rope_theta=500000.0, b_sigma=0.2,
                           name="graph prefill")
    pd = PrefillDev(pcase)
    p_out = torch.empty_like(pd.q)
    n_tok, d_model, r = 300, 4096, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(93)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x = torch.empty((n_tok, d_model), **bf)
    a_k = (torch.randn((r, d_model), generator=g, device="cuda") / 64).to(torch.bfloat16)
    a_v = (torch.randn((r, d_model), generator=g, device="cuda") / 64).to(torch.bfloat16)
    l_k = torch.zeros((n_tok, r), **bf)
    l_v = torch.zeros((n_tok, r), **bf)
    lr_ws = torch.zeros(max(16, lra.lr_cache_build_workspace_size(
        dtype=1, n_tok=n_tok, d_model=d_model, rank=r)), dtype=torch.uint8, device="cuda")
    assert lr_ws.numel() > 16

    def step():
        lra.lr_cache_build(x, a_k, a_v, l_k, l_v, workspace=lr_ws)
        pd.run(out=p_out)
        dd.run(out=d_out, workspace=d_ws)

    def inputs(i):
        gi = torch.Generator(device="cuda")
        gi.manual_seed(1000 + i)
        return (torch.randn(dd.q.shape, generator=gi, device="cuda").to(torch.bfloat16),
                torch.randn(pd.q.shape, generator=gi, device="cuda").to(torch.bfloat16),
                torch.randn(x.shape, generator=gi, device="cuda").to(torch.bfloat16))

    def load(i):
        qd, qp, xi = inputs(i)
        dd.q.copy_(qd)
        pd.q.copy_(qp)
        x.copy_(xi)

    def results():
        return [t.clone() for t in (d_out, p_out, l_k, l_v)]

    refs = []
    for i in range(3):
        load(i)
        step()
        torch.cuda.synchronize()
        refs.append(results())
    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rnd in range(2):
        for i in range(3):
            load(i)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = results()
            for name, a, b in zip(("decode", "prefill", "L_k", "L_v"), got, refs[i]):
                assert torch.equal(a, b), f"replay {rnd}/{i}: {name} differs from the eager call"
            # eager work between replays on the same buffers
            step()
            torch.cuda.synchronize()
            for name, a, b in zip(("decode", "prefill", "L_k", "L_v"), results(), refs[i]):
                assert torch.equal(a, b), f"eager after replay {rnd}/{i}: {name} differs"
    # the decode workspace's per-unit counters and queue words are back at zero
    n_units = 2 * 8
    assert int(d_ws[:4 * (n_units + 2)].view(torch.int32).abs().sum()) == 0


def test_concurrent_streams_equal_sequential():
    """Two decode calls with their own workspaces on two streams (default priority) running at
    the same time give the bits of the same calls run one after the other: the library keeps no
    global mutable state between calls."""
    import torch
    import attention_shared_base_amd as lra
    cases = [w.make_decode(95 + i, dtype="bf16", ctx_lens=[4000, 2500], reqs=[(0, 0), (0, 1), (1, 1)],
                           n_agents=2, h_q=32, h_kv=8, d=128, r=16, shuffle=True, name=f"stream {i}")
             for i in range(2)]
    devs = [DecodeDev(c) for c in cases]
    wss = [torch.zeros(lra.decode_workspace_size(
        n_q_heads=32, n_kv_heads=8, head_dim=128, rank=16, dtype=1, n_req=3, n_ctx=2,
        max_req_per_ctx=d.max_req_per_ctx, max_ctx_len=d.max_ctx_len), dtype=torch.uint8,
        device="cuda") for d in devs]
    outs = [torch.empty_like(d.q) for d in devs]
    for d, o, ws in zip(devs, outs, wss):
        d.run(out=o, workspace=ws)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for d, o, ws, st in zip(devs, outs, wss, streams):
            with torch.cuda.stream(st):
                for _ in range(3):
                    d.run(out=o, workspace=ws)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), f"stream {i}, round {rep}"
