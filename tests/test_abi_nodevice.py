"""C-ABI behaviour on a machine without a GPU: every launching entry point, given valid
scalars, passes validation and then reports LRA_ERR_HIP (with detail text) instead of
crashing; and random scalar arguments never crash the validation layer (property test).

These calls pass fake (aligned, non-null) device pointers, so they are skipped whenever a
GPU is visible: there the launches would dereference them."""
import ctypes
import os

import pytest

import attention_shared_base_amd as lra

pytestmark = pytest.mark.skipif(not os.path.exists(lra.lib_path),
                                reason="liblra_attn.so not built (run __graft_entry__.build())")

OK, NULL_PTR, BAD_SHAPE, UNSUPPORTED, MISALIGNED, WS_SMALL, HIP = range(7)
A = ctypes.c_void_p(0x100000)  # fake, 16-byte aligned


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0  # counts devices without initialising one


needs_no_gpu = pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: only without a GPU")


def dims(h_q=32, h_kv=8, d=128, r=16, dt=1, scale=0.0, stride=0):
    return lra.Dims(h_q, h_kv, d, r, dt, scale, stride)


def _err(lib):
    return lib.lra_last_error().decode()


@needs_no_gpu
def test_launching_entry_points_report_hip_error():
    lib = lra.load()
    dm = dims()
    cases = {
        "rope_table": lambda: lib.lra_rope_table_build(ctypes.c_double(5e5), 128, 64, A, A, None),
        "prefill": lambda: lib.lra_attn_prefill(ctypes.byref(dm), A, 2, 16, A, A, A, 64, A, A, A, A, 2,
                                                None, None, 0, A, None),
        "prefill_rope": lambda: lib.lra_attn_prefill(ctypes.byref(dm), A, 2, 16, A, A, A, 64, A, A, A, A, 2,
                                                     A, A, 64, A, None),
        "prefill_f32": lambda: lib.lra_attn_prefill(ctypes.byref(dims(dt=0)), A, 2, 16, A, A, A, 64, A, A, A,
                                                    A, 2, None, None, 0, A, None),
        "prefill_paged": lambda: lib.lra_attn_prefill_paged(ctypes.byref(dm), A, 2, 16, A, A, A, A, A, 8, 16,
                                                            A, 4, 64, A, A, 2, None, None, 0, A, None),
        "decode": lambda: lib.lra_attn_decode(ctypes.byref(dm), A, 4, A, 1, 4, A, A, A, A, A, 8, 16, A, 4, A,
                                              64, A, A, 4, None, None, 0, A, A, 1 << 20, None),
        "decode_noalloc": lambda: lib.lra_attn_decode_noalloc(ctypes.byref(dm), A, 4, A, 1, 4, A, A, A, A, A, 8,
                                                              16, A, 4, A, 64, A, A, 4, None, None, 0, A, None),
        "lr_build": lambda: lib.lra_lr_cache_build(1, A, 64, 4096, A, A, 16, 1, A, A, 0, 0, None, 0, None),
        "append": lambda: lib.lra_cache_append(ctypes.byref(dm), 4, A, A, A, A, A, 1, A, A, A, A, 8, 16, None),
        "naive_expand": lambda: lib.lra_naive_expand_pages(ctypes.byref(dm), 4, A, 1, A, A, A, A, A, 8, 16, A, 4,
                                                           A, A, A, 4, A, A, 4, None),
        "ceiling_read": lambda: lib.lra_ceiling_hbm_read(A, 1 << 20, 0, 1, A, None),
        "ceiling_mfma": lambda: lib.lra_ceiling_mfma_bf16(1, 256, 16, A, None),
    }
    for name, call in cases.items():
        st = call()
        assert st == HIP, f"{name}: status {st} ({_err(lib)})"
        assert _err(lib), name


@needs_no_gpu
def test_random_scalars_never_crash_the_validation():
    """Random shapes, sizes, strides and null / misaligned pointers: every call returns one
    of the documented statuses (on this machine a call that passes validation fails at the
    launch with LRA_ERR_HIP, or returns LRA_OK when there is nothing to do)."""
    hypothesis = pytest.importorskip("hypothesis")
    st_ = hypothesis.strategies
    lib = lra.load()
    ptrs = st_.sampled_from([A, A, A, None, ctypes.c_void_p(0x100004)])
    ints = st_.integers(min_value=-3, max_value=70000)
    small = st_.integers(min_value=-2, max_value=40)

    @hypothesis.settings(max_examples=400, deadline=None, derandomize=True)
    @hypothesis.given(h_q=small, h_kv=small, d=st_.sampled_from([0, 32, 64, 96, 128, 256]),
                      r=st_.sampled_from([0, 2, 4, 8, 12, 16, 32, 64]), dt=st_.integers(-1, 2),
                      stride=st_.sampled_from([0, -1, 1, 1 << 20, 1 << 40]), n_req=small, q_len=ints,
                      kv_len=ints, n_agents=small, page=st_.sampled_from([8, 16, 32]), max_blocks=ints,
                      n_pages=ints, rows=ints, p=ptrs, rope=st_.booleans())
    def check(h_q, h_kv, d, r, dt, stride, n_req, q_len, kv_len, n_agents, page, max_blocks, n_pages, rows,
              p, rope):
        dm = lra.Dims(h_q, h_kv, d, r, dt, 0.0, stride)
        cs = (A, A) if rope else (None, None)
        codes = (
            lib.lra_attn_prefill(ctypes.byref(dm), p, n_req, q_len, A, A, A, kv_len, A, A, A, A, n_agents,
                                 cs[0], cs[1], rows, A, None),
            lib.lra_attn_prefill_paged(ctypes.byref(dm), A, n_req, q_len, A, A, A, A, p, n_pages, page, A,
                                       max_blocks, kv_len, A, A, n_agents, cs[0], cs[1], rows, A, None),
            lib.lra_attn_decode(ctypes.byref(dm), A, n_req, A, max(n_agents, 0) % 8, 4, A, A, A, A, p,
                                n_pages, page, A, max_blocks, A, kv_len, A, A, n_agents, cs[0], cs[1], rows,
                                A, A, 1 << 30, None),
            lib.lra_cache_append(ctypes.byref(dm), n_req, A, A, A, A, A, n_agents, A, A, A, p, n_pages, page,
                                 None),
        )
        for c in codes:
            assert c in (OK, NULL_PTR, BAD_SHAPE, UNSUPPORTED, MISALIGNED, WS_SMALL, HIP), c
        size = lib.lra_attn_decode_workspace_size(ctypes.byref(dm), n_req, max(n_agents, 1), 4, kv_len)
        assert size >= 0

    check()
