"""C-ABI checks that need no GPU: the library loads, exports every declared entry
point, and rejects bad scalar arguments before touching the device."""
import ctypes
import os
import re

import pytest

import attention_shared_base_amd as lra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lra_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lra.lib_path),
                                reason="liblra_attn.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lra_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(lra.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(lra.lib_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = lra.load()
    assert lra.abi_version() == 6
    for s in range(7):
        assert lib.lra_status_str(s).decode().startswith("LRA_")
    assert b"unknown" in lib.lra_status_str(99)


# Fake but 16-byte-aligned non-null addresses: validation must fail before any use.
A = ctypes.c_void_p(0x100000)


def dims(h_q=32, h_kv=8, d=128, r=16, dt=1, scale=0.0, stride=0):
    return lra.Dims(h_q, h_kv, d, r, dt, scale, stride)


def call_decode(dm, **over):
    lib = lra.load()
    # 4 contexts x 8192 tokens, 4 requests each: several chunks per unit, so the
    # call needs a workspace and every case below fails validation before launch.
    args = dict(q=A, n_req=16, crs=A, n_ctx=4, mrpc=4, agent=A, k=A, v=A, lk=A, lv=A,
                n_pages=2048, page=16, bt=A, max_blocks=512, clen=A, max_ctx=8192, bk=A, bv=A,
                n_agents=4, cos=None, sin=None, rows=8192, out=A, ws=A, ws_bytes=1 << 30)
    args.update(over)
    st = lib.lra_attn_decode(ctypes.byref(dm), args["q"], args["n_req"], args["crs"], args["n_ctx"],
                             args["mrpc"], args["agent"], args["k"], args["v"], args["lk"],
                             args["lv"], args["n_pages"], args["page"], args["bt"],
                             args["max_blocks"], args["clen"], args["max_ctx"], args["bk"],
                             args["bv"], args["n_agents"], args["cos"], args["sin"], args["rows"],
                             args["out"], args["ws"], args["ws_bytes"], None)
    return st, lib.lra_last_error().decode()


@pytest.mark.parametrize("dm,over,want", [
    (dims(d=96), {}, 3),
    (dims(r=2), {}, 3),
    (dims(r=12), {}, 3),
    (dims(dt=2), {}, 3),
    (dims(h_q=30, h_kv=8), {}, 2),
    (dims(h_q=0), {}, 2),
    (dims(h_q=64, h_kv=2), {}, 3),          # g = 32 > 16 rows of one bf16 tile
    (dims(scale=float("nan")), {}, 2),
    (dims(), {"page": 32}, 3),
    (dims(), {"n_req": -1}, 2),
    (dims(), {"n_ctx": 0}, 2),
    (dims(), {"mrpc": 0}, 2),
    (dims(), {"mrpc": 17}, 2),
    (dims(), {"n_pages": 0}, 2),
    (dims(), {"max_ctx": 8193}, 2),          # > max_blocks * page
    (dims(), {"max_ctx": -1}, 2),
    (dims(), {"n_agents": 0}, 2),
    (dims(), {"q": None}, 1),
    (dims(), {"bt": None}, 1),
    (dims(), {"out": None}, 1),
    (dims(), {"k": ctypes.c_void_p(0x100008)}, 4),
    (dims(), {"ws_bytes": 1}, 5),
    (dims(), {"ws": None}, 1),
    (dims(), {"cos": A}, 1),                 # rope tables go in pairs
    (lra.Dims(32, 8, 128, 16, 1, 0.0, -1), {}, 2),   # negative LR stride
    # per-agent LR + RoPE is supported: a short table is still rejected before launch
    (lra.Dims(32, 8, 128, 16, 1, 0.0, 2048 * 16 * 16), {"cos": A, "sin": A, "rows": 100}, 2),
    (dims(), {"cos": A, "sin": ctypes.c_void_p(0x100004)}, 4),
    (dims(), {"cos": A, "sin": A, "rows": 8191}, 2),          # tables shorter than max_ctx_len
    (dims(), {"cos": A, "sin": A, "rows": 0, "max_ctx": 0}, 2),  # at least one row
    # one LR pool per agent: the stride must cover n_pages * page * r elements
    (lra.Dims(32, 8, 128, 16, 1, 0.0, 2048 * 16 * 16 - 1), {}, 2),
])
def test_decode_validation(dm, over, want):
    st, msg = call_decode(dm, **over)
    assert st == want, msg
    assert msg


def test_decode_null_dims():
    lib = lra.load()
    st = lib.lra_attn_decode(None, A, 1, A, 1, 1, A, A, A, A, A, 1, 16, A, 1, A, 16, A, A, 1, None,
                             None, 0, A, A, 0, None)
    assert st == 1


def call_prefill(dm, **over):
    lib = lra.load()
    a = dict(q=A, n_req=2, q_len=16, agent=A, k=A, v=A, kv_len=256, lk=A, lv=A, bk=A, bv=A,
             n_agents=2, cos=None, sin=None, rows=256, out=A)
    a.update(over)
    st = lib.lra_attn_prefill(ctypes.byref(dm), a["q"], a["n_req"], a["q_len"], a["agent"], a["k"],
                              a["v"], a["kv_len"], a["lk"], a["lv"], a["bk"], a["bv"],
                              a["n_agents"], a["cos"], a["sin"], a["rows"], a["out"], None)
    return st, lib.lra_last_error().decode()


@pytest.mark.parametrize("over,want", [
    ({"q_len": 0}, 2),
    ({"kv_len": 15}, 2),
    ({"n_agents": 0}, 2),
    ({"cos": A}, 1),
    ({"v": None}, 1),
    ({"lk": ctypes.c_void_p(0x100004)}, 4),
    ({"n_req": -3}, 2),
    ({"cos": A, "sin": A, "rows": 255}, 2),   # RoPE tables shorter than kv_len
])
def test_prefill_validation(over, want):
    st, msg = call_prefill(dims(), **over)
    assert st == want, msg


def test_prefill_per_agent_stride():
    # one LR cache per agent: the stride must cover kv_len * r elements
    st, msg = call_prefill(lra.Dims(32, 8, 128, 16, 1, 0.0, 256 * 16 - 1))
    assert st == 2 and "lr_agent_stride" in msg


def test_prefill_zero_requests_is_a_no_op():
    assert call_prefill(dims(), n_req=0)[0] == 0


def test_lr_build_validation():
    lib = lra.load()

    def call(**o):
        a = dict(dt=1, x=A, n_tok=16, d_model=4096, ak=A, av=A, r=16, n_lr=1, lk=A, lv=A, off=0,
                 ls=0, ws=None, wsz=0)
        a.update(o)
        return lib.lra_lr_cache_build(a["dt"], a["x"], a["n_tok"], a["d_model"], a["ak"], a["av"],
                                      a["r"], a["n_lr"], a["lk"], a["lv"], a["off"], a["ls"],
                                      a["ws"], a["wsz"], None)

    assert call(r=12) == 3
    assert call(r=2) == 3
    assert call(dt=5) == 3
    assert call(d_model=100) == 3
    assert call(d_model=0) == 2
    assert call(n_tok=-1) == 2
    assert call(off=-1) == 2
    assert call(x=None) == 1
    assert call(av=ctypes.c_void_p(0x100002)) == 4
    assert call(n_tok=0) == 0
    assert call(n_lr=0) == 2
    assert call(n_lr=4, ls=16 * 16 - 1) == 2      # agents' caches would overlap
    assert call(n_lr=4, ls=16 * 16, n_tok=0) == 0
    # a workspace that is given must be large enough and aligned (16 tokens: split in 8)
    need = lra.lr_cache_build_workspace_size(dtype=1, n_tok=16, d_model=4096, rank=16)
    assert need > 0
    assert call(ws=A, wsz=need - 1) == 5
    assert call(ws=ctypes.c_void_p(0x100008), wsz=need) == 4


def test_rope_table_validation():
    lib = lra.load()
    assert lib.lra_rope_table_build(-1.0, 128, 10, A, A, None) == 2
    assert lib.lra_rope_table_build(1e4, 127, 10, A, A, None) == 2
    assert lib.lra_rope_table_build(1e4, 128, 10, None, A, None) == 1
    assert lib.lra_rope_table_build(1e4, 128, 0, A, A, None) == 0


def test_workspace_size_queries():
    lib = lra.load()
    dm = dims()
    # 4 contexts x 8192 tokens, 4 requests each: split into several chunks -> workspace needed
    ws = lib.lra_attn_decode_workspace_size(ctypes.byref(dm), 16, 4, 4, 8192)
    assert ws > 0
    # the workspace grows with (d + r + 2) floats per partial row, never with kv_len * d
    ws_small = lib.lra_attn_decode_workspace_size(ctypes.byref(dm), 16, 4, 4, 128)
    assert ws_small == 0  # a single chunk per unit needs no partials
    assert lib.lra_attn_decode_workspace_size(ctypes.byref(dims(dt=0)), 16, 4, 4, 8192) == 0
    assert lib.lra_attn_decode_workspace_size(ctypes.byref(dims(d=96)), 16, 4, 4, 8192) == 0


def call_expand(dm, **over):
    lib = lra.load()
    a = dict(n_req=4, crs=A, n_ctx=2, agent=A, k=A, v=A, lk=A, lv=A, n_pages=64, page=16, bt=A,
             max_blocks=32, clen=A, bk=A, bv=A, n_agents=2, ko=A, vo=A, out_blocks=32)
    a.update(over)
    st = lib.lra_naive_expand_pages(ctypes.byref(dm), a["n_req"], a["crs"], a["n_ctx"], a["agent"],
                                    a["k"], a["v"], a["lk"], a["lv"], a["n_pages"], a["page"],
                                    a["bt"], a["max_blocks"], a["clen"], a["bk"], a["bv"],
                                    a["n_agents"], a["ko"], a["vo"], a["out_blocks"], None)
    return st, lib.lra_last_error().decode()


@pytest.mark.parametrize("dm,over,want", [
    (dims(dt=0), {}, 3),                     # the baseline is bf16 only
    (dims(r=2), {}, 3),
    (dims(r=12), {}, 3),
    (dims(), {"page": 8}, 3),
    (dims(), {"out_blocks": 0}, 2),
    (dims(), {"out_blocks": 33}, 2),
    (dims(), {"n_ctx": 0}, 2),
    (dims(), {"ko": None}, 1),
    (dims(), {"vo": ctypes.c_void_p(0x100002)}, 4),
    (dims(stride=64 * 16 * 16 - 1), {}, 2),   # per-agent LR pools: stride below one pool
])
def test_naive_expand_validation(dm, over, want):
    st, msg = call_expand(dm, **over)
    assert st == want, msg
    assert msg


def test_paged_prefill_and_append_validation():
    lib = lra.load()
    dm = dims()
    # the staged path's workspace grows with kv_len and is 0 for an invalid dims
    assert lib.lra_attn_prefill_paged_staged_workspace_size(ctypes.byref(dm), 1000) > \
        lib.lra_attn_prefill_paged_staged_workspace_size(ctypes.byref(dm), 10) > 0
    assert lib.lra_attn_prefill_paged_staged_workspace_size(ctypes.byref(dims(dt=0)), 10) == 0

    base = dict(q=A, n_req=2, q_len=16, agent=A, k=A, v=A, lk=A, lv=A, n_pages=64, page=16, bt=A,
                max_blocks=16, kv_len=256, bk=A, bv=A, n_agents=2, cos=None, sin=None, rows=256,
                out=A, ws=A, ws_bytes=1 << 30)

    def pp(**o):  # direct: reads the pages in place, no workspace
        a = dict(base, **o)
        return lib.lra_attn_prefill_paged(ctypes.byref(o.pop("dm", dm)), a["q"], a["n_req"], a["q_len"],
                                          a["agent"], a["k"], a["v"], a["lk"], a["lv"], a["n_pages"],
                                          a["page"], a["bt"], a["max_blocks"], a["kv_len"], a["bk"],
                                          a["bv"], a["n_agents"], a["cos"], a["sin"], a["rows"],
                                          a["out"], None)

    def ps(**o):  # staged through a contiguous copy
        a = dict(base, **o)
        return lib.lra_attn_prefill_paged_staged(
            ctypes.byref(o.pop("dm", dm)), a["q"], a["n_req"], a["q_len"], a["agent"], a["k"], a["v"],
            a["lk"], a["lv"], a["n_pages"], a["page"], a["bt"], a["max_blocks"], a["kv_len"], a["bk"],
            a["bv"], a["n_agents"], a["cos"], a["sin"], a["rows"], a["out"], a["ws"], a["ws_bytes"], None)
    for f in (pp, ps):
        assert f(max_blocks=15) == 2            # 15 blocks cannot hold 256 tokens
        assert f(kv_len=8) == 2                  # kv_len < q_len
        assert f(page=32) == 3
        assert f(cos=A) == 1
        assert f(cos=A, sin=A, rows=255) == 2    # RoPE tables shorter than kv_len
        assert f(bt=None) == 1
        assert f(n_pages=0) == 2
        assert f(dm=dims(dt=0)) == 3             # bf16 only
    assert ps(ws_bytes=1) == 5
    assert ps(ws=None) == 1
    # per-agent LR pools: the direct path takes them (stride >= one agent's pool), the
    # staged path does not
    assert pp(dm=dims(stride=64 * 16 * 16 - 1)) == 2
    assert ps(dm=dims(stride=64 * 16 * 16)) == 3

    def ap(**o):
        a = dict(n=4, slots=A, k=A, v=A, lk=A, lv=A, n_lr=1, kp=A, vp=A, lkp=A, lvp=A, n_pages=8, page=16)
        a.update(o)
        return lib.lra_cache_append(ctypes.byref(o.pop("dm", dm)), a["n"], a["slots"], a["k"], a["v"],
                                    a["lk"], a["lv"], a["n_lr"], a["kp"], a["vp"], a["lkp"], a["lvp"],
                                    a["n_pages"], a["page"], None)
    assert ap(slots=None) == 1
    assert ap(n=-1) == 2
    assert ap(page=8) == 3
    assert ap(dm=dims(dt=0)) == 3
    assert ap(kp=ctypes.c_void_p(0x100004)) == 4
    assert ap(n_lr=0) == 2
    assert ap(n_lr=2) == 2                                  # several row sets need per-agent pools
    assert ap(n_lr=2, dm=dims(stride=8 * 16 * 16 - 1)) == 2  # stride below one agent's pool


def test_lr_build_workspace_size():
    """Split plan: ranges of d_model until one agent's token blocks cover 256 CUs, each
    range >= 16 slices;
    partials of 64 tokens x 2r fp32 per range, counters padded to 256 bytes."""
    ws = lambda **o: lra.lr_cache_build_workspace_size(**{**dict(dtype=1, d_model=4096, rank=16), **o})
    # 4096 tokens: 64 blocks x 4 ranges = 256 workgroups
    assert ws(n_tok=4096) == 256 + 64 * 4 * 64 * 32 * 4
    # 16384 tokens fill the GPU without a split: no workspace
    assert ws(n_tok=16384) == 0
    # 8 agents x 1024 tokens: the split of one agent's 16 blocks (8 ranges), 128 units
    assert ws(n_tok=1024, n_lr=8) == 512 + 128 * 8 * 64 * 32 * 4
    # at most 8 ranges, and d_model 1024 (32 slices) allows only 2
    assert ws(n_tok=64) == 256 + 1 * 8 * 64 * 32 * 4
    assert ws(n_tok=64, d_model=1024) == 256 + 1 * 2 * 64 * 32 * 4
    assert ws(n_tok=4096, rank=32) == 256 + 64 * 4 * 64 * 64 * 4
    # fp32 and rejected arguments need none
    assert ws(n_tok=4096, dtype=0) == 0
    assert ws(n_tok=4096, rank=12) == 0
    # rank 4: partial rows padded to one 16-column tile
    assert ws(n_tok=4096, rank=4) == 256 + 64 * 4 * 64 * 16 * 4
    assert ws(n_tok=0) == 0


def test_decode_noalloc_limits_and_dtype():
    """The allocation-free decode rejects, before any HIP call, problems whose split-K
    partials exceed its fixed scratch, and the fp32 path (which needs none)."""
    lib = lra.load()
    dm = dims()

    def call(dm_, n_ctx, mrpc, max_ctx):
        return lib.lra_attn_decode_noalloc(ctypes.byref(dm_), A, n_ctx * mrpc, A, n_ctx, mrpc, A, A,
                                           A, A, A, 1 << 20, 16, A, 1 << 16, A, max_ctx, A, A, 4,
                                           None, None, 0, A, None)
    # 1024 contexts x 64k tokens: 8192 units x 16 chunks of partials (about 1.3 GB)
    assert call(dm, 1024, 1, 65536) == 5
    assert "scratch" in lib.lra_last_error().decode()
    assert call(dims(dt=0), 1, 1, 256) == 3
    assert call(dims(d=96), 1, 1, 256) == 3


def test_naive_prefill_validation():
    lib = lra.load()
    dm = dims()
    need = lib.lra_naive_prefill_workspace_size(ctypes.byref(dm), 4, 1000)
    assert need == 2 * 4 * 8 * 1000 * 128 * 2
    assert lib.lra_naive_prefill_workspace_size(ctypes.byref(dims(dt=0)), 4, 1000) == 0

    def call(dm_=dm, **o):
        a = dict(q=A, n_req=2, q_len=16, agent=A, k=A, v=A, kv_len=256, lk=A, lv=A, bk=A, bv=A,
                 n_agents=2, cos=None, sin=None, rows=256, out=A, ws=A, wsz=1 << 30)
        a.update(o)
        return lib.lra_naive_prefill(ctypes.byref(dm_), a["q"], a["n_req"], a["q_len"], a["agent"],
                                     a["k"], a["v"], a["kv_len"], a["lk"], a["lv"], a["bk"], a["bv"],
                                     a["n_agents"], a["cos"], a["sin"], a["rows"], a["out"], a["ws"],
                                     a["wsz"], None)
    assert call(dims(dt=0)) == 3
    assert call(q_len=0) == 2
    assert call(kv_len=8) == 2
    assert call(ws=None) == 1
    assert call(wsz=16) == 5
    assert call(cos=A, sin=A, rows=255) == 2
    assert call(n_req=0) == 0


def test_ceiling_validation():
    lib = lra.load()
    rd = lib.lra_ceiling_hbm_read
    assert rd(None, 1024, 0, 1, A, None) == 1
    assert rd(A, 1024, 0, 1, None, None) == 1
    assert rd(ctypes.c_void_p(0x100008), 1024, 0, 1, A, None) == 4
    assert rd(A, 0, 0, 1, A, None) == 2
    assert rd(A, 1000, 0, 1, A, None) == 2
    assert rd(A, 1024, -1, 1, A, None) == 2
    assert rd(A, 1024, 65536, 1, A, None) == 2
    assert rd(A, 1024, 0, 4, A, None) == 2
    assert rd(A, 1024, 0, -1, A, None) == 2
    mm = lib.lra_ceiling_mfma_bf16
    assert mm(0, 256, 16, None, None) == 1
    assert mm(3, 256, 16, A, None) == 2
    assert mm(-1, 256, 16, A, None) == 2
    assert mm(0, 0, 16, A, None) == 2
    assert mm(1, 65536, 16, A, None) == 2
    assert mm(0, 256, 0, A, None) == 2
    assert mm(0, 256, (1 << 20) + 1, A, None) == 2
