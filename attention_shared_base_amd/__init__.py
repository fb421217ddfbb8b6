"""Flash-LoRA-Attention for AMD MI355X (gfx950): thin Python binding.

Multi-LoRA agents share a base KV cache and a low-rank (LR) cache and apply
their own up-projections B_k, B_v (LRAgent, arXiv 2602.01053v2, §3 and App. B;
PReCache, arXiv 2609.34054, PreLRShared).  All arithmetic runs in the HIP
kernels of ``liblra_attn.so`` (C ABI in ``include/lra_attn.h``); this module
only marshals torch tensors (device memory) and the current HIP stream into
those calls.  There is no CPU fallback: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LraError", "lib_path", "load", "decode", "decode_workspace_size", "prefill",
    "lr_cache_build", "lr_cache_build_workspace_size", "rope_table", "abi_version", "EXPORTED_SYMBOLS", "naive_decode",
    "prefill_paged", "prefill_paged_staged", "prefill_paged_staged_workspace_size",
    "cache_append", "decode_noalloc", "prepare_decode", "prepare_prefill", "PreparedCall",
    "naive_prefill", "naive_prefill_workspace_size", "ceiling_hbm_read", "ceiling_mfma_bf16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "liblra_attn.so")

LRA_F32, LRA_BF16 = 0, 1
ABI_VERSION = 6  # LRA_ABI_VERSION of include/lra_attn.h

EXPORTED_SYMBOLS = (
    "lra_abi_version", "lra_status_str", "lra_last_error", "lra_attn_decode_workspace_size",
    "lra_attn_decode", "lra_attn_prefill", "lra_lr_cache_build",
    "lra_lr_cache_build_workspace_size", "lra_rope_table_build",
    "lra_naive_expand_pages", "lra_attn_prefill_paged", "lra_attn_prefill_paged_staged_workspace_size",
    "lra_attn_prefill_paged_staged",
    "lra_cache_append", "lra_attn_decode_noalloc", "lra_naive_prefill_workspace_size",
    "lra_naive_prefill", "lra_ceiling_hbm_read", "lra_ceiling_mfma_bf16",
)


class LraError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"status {status}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("lr_agent_stride", ctypes.c_int64)]


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32


def load():
    """Load liblra_attn.so once; raises if it has not been built.

    torch is imported first: its HIP runtime (``libamdhip64.so``, soname
    ``libamdhip64.so.7``) then satisfies the library's dependency, so the process
    holds one HIP runtime.  Loaded the other way round, the library would bring in
    the system runtime and torch a second one, and launches on torch's memory
    would find no device."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} not found: build it with "
                          "`python -m attention_shared_base_amd.build` (hipcc, gfx950)")
    import torch  # noqa: F401  (one HIP runtime per process: torch's)
    lib = ctypes.CDLL(lib_path)
    lib.lra_abi_version.restype = I32
    lib.lra_abi_version.argtypes = []
    if lib.lra_abi_version() != ABI_VERSION:
        raise ImportError(f"{lib_path} has ABI {lib.lra_abi_version()}, this binding expects "
                          f"{ABI_VERSION}: rebuild it")
    lib.lra_status_str.restype = ctypes.c_char_p
    lib.lra_status_str.argtypes = [I32]
    lib.lra_last_error.restype = ctypes.c_char_p
    lib.lra_last_error.argtypes = []
    lib.lra_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.lra_attn_decode_workspace_size.argtypes = [ctypes.POINTER(Dims), I32, I32, I32, I32]
    lib.lra_attn_decode.restype = I32
    lib.lra_attn_decode.argtypes = [
        ctypes.POINTER(Dims), P, I32, P, I32, I32, P, P, P, P, P, I32, I32, P, I32, P, I32,
        P, P, I32, P, P, I32, P, P, ctypes.c_size_t, P]
    lib.lra_attn_decode_noalloc.restype = I32
    lib.lra_attn_decode_noalloc.argtypes = [
        ctypes.POINTER(Dims), P, I32, P, I32, I32, P, P, P, P, P, I32, I32, P, I32, P, I32,
        P, P, I32, P, P, I32, P, P]
    lib.lra_attn_prefill.restype = I32
    lib.lra_attn_prefill.argtypes = [
        ctypes.POINTER(Dims), P, I32, I32, P, P, P, I32, P, P, P, P, I32, P, P, I32, P, P]
    lib.lra_lr_cache_build.restype = I32
    lib.lra_lr_cache_build.argtypes = [I32, P, I32, I32, P, P, I32, I32, P, P, ctypes.c_int64,
                                       ctypes.c_int64, P, ctypes.c_size_t, P]
    lib.lra_lr_cache_build_workspace_size.restype = ctypes.c_size_t
    lib.lra_lr_cache_build_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.lra_rope_table_build.restype = I32
    lib.lra_rope_table_build.argtypes = [ctypes.c_double, I32, I32, P, P, P]
    lib.lra_attn_prefill_paged.restype = I32
    lib.lra_attn_prefill_paged.argtypes = [
        ctypes.POINTER(Dims), P, I32, I32, P, P, P, P, P, I32, I32, P, I32, I32, P, P, I32, P, P,
        I32, P, P]
    lib.lra_attn_prefill_paged_staged_workspace_size.restype = ctypes.c_size_t
    lib.lra_attn_prefill_paged_staged_workspace_size.argtypes = [ctypes.POINTER(Dims), I32]
    lib.lra_attn_prefill_paged_staged.restype = I32
    lib.lra_attn_prefill_paged_staged.argtypes = [
        ctypes.POINTER(Dims), P, I32, I32, P, P, P, P, P, I32, I32, P, I32, I32, P, P, I32, P, P,
        I32, P, P, ctypes.c_size_t, P]
    lib.lra_cache_append.restype = I32
    lib.lra_cache_append.argtypes = [ctypes.POINTER(Dims), I32, P, P, P, P, P, I32, P, P, P, P, I32,
                                     I32, P]
    lib.lra_naive_prefill_workspace_size.restype = ctypes.c_size_t
    lib.lra_naive_prefill_workspace_size.argtypes = [ctypes.POINTER(Dims), I32, I32]
    lib.lra_naive_prefill.restype = I32
    lib.lra_naive_prefill.argtypes = [
        ctypes.POINTER(Dims), P, I32, I32, P, P, P, I32, P, P, P, P, I32, P, P, I32, P, P,
        ctypes.c_size_t, P]
    lib.lra_naive_expand_pages.restype = I32
    lib.lra_naive_expand_pages.argtypes = [
        ctypes.POINTER(Dims), I32, P, I32, P, P, P, P, P, I32, I32, P, I32, P, P, P, I32, P, P,
        I32, P]
    lib.lra_ceiling_hbm_read.restype = I32
    lib.lra_ceiling_hbm_read.argtypes = [P, ctypes.c_size_t, I32, I32, P, P]
    lib.lra_ceiling_mfma_bf16.restype = I32
    lib.lra_ceiling_mfma_bf16.argtypes = [I32, I32, I32, P, P]
    _lib = lib
    return lib


def abi_version():
    return int(load().lra_abi_version())


def _check(status):
    if status != 0:
        lib = load()
        raise LraError(status, f"{lib.lra_status_str(status).decode()} — {lib.lra_last_error().decode()}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return LRA_BF16
    if t.dtype == torch.float32:
        return LRA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows(t):
    return 0 if t is None else int(t.shape[0])


def _stream(t, stream):
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _contig(name, t):
    _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(t.device.type == "cuda", f"{name} must be a device tensor")
    return t


def _dims(h_q, h_kv, d, r, dtype, scale, lr_stride=0):
    return Dims(h_q, h_kv, d, r, dtype, float(scale), int(lr_stride))


def decode_workspace_size(*, n_q_heads, n_kv_heads, head_dim, rank, dtype, n_req, n_ctx,
                          max_req_per_ctx, max_ctx_len, lr_agent_stride=0):
    dims = _dims(n_q_heads, n_kv_heads, head_dim, rank, dtype, 0.0, lr_agent_stride)
    return int(load().lra_attn_decode_workspace_size(ctypes.byref(dims), n_req, n_ctx,
                                                      max_req_per_ctx, max_ctx_len))


def decode(q, ctx_req_start, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table, ctx_len,
           b_k, b_v, *, max_req_per_ctx, max_ctx_len, rope_cos=None, rope_sin=None, out=None,
           workspace=None, softmax_scale=0.0, stream=None, _prepare=False):
    """Paged decode (``lra_attn_decode``).  Layouts as in include/lra_attn.h:

    q [n_req, H_q, d]; k_pool [n_pages, H_kv, d/8, 16, 8]; v_pool [n_pages, H_kv, d, 16];
    lk_pool [n_pages, 16, r]; lv_pool [n_pages, r, 16] (one LR cache for every agent) or
    [n_agents, n_pages, 16, r] / [n_agents, n_pages, r, 16] (one per agent);
    block_table [n_ctx, max_blocks];
    ctx_len [n_ctx]; ctx_req_start [n_ctx+1]; req_agent [n_req]; b_k, b_v [n_agents, r, H_kv*d];
    optional RoPE tables rope_cos, rope_sin [>= max(max_ctx_len, 1), d/2] fp32 rotate the
    adapter key term.  ``workspace`` (uint8, zero-filled before first use) is allocated
    when not given.
    """
    import torch
    lib = load()
    n_req, h_q, d = q.shape
    n_pages, h_kv, d8, page, eight = k_pool.shape
    _need(d8 * 8 == d and eight == 8, "k_pool must be [n_pages, H_kv, d/8, page, 8]")
    r = lk_pool.shape[-1]
    n_ctx, max_blocks = block_table.shape
    n_agents = b_k.shape[0]
    per_agent = lk_pool.dim() == 4
    lr_stride = n_pages * page * r if per_agent else 0
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("lk_pool", lk_pool),
                    ("lv_pool", lv_pool), ("b_k", b_k), ("b_v", b_v)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from q")
    for name, t in (("ctx_req_start", ctx_req_start), ("req_agent", req_agent),
                    ("block_table", block_table), ("ctx_len", ctx_len)):
        _contig(name, t)
        _need(t.dtype == torch.int32, f"{name} must be int32")
    _need(tuple(v_pool.shape) == (n_pages, h_kv, d, page), "v_pool must be [n_pages, H_kv, d, page]")
    lead = (n_agents,) if per_agent else ()
    _need(tuple(lk_pool.shape) == lead + (n_pages, page, r), "lk_pool must be [(n_agents,) n_pages, page, r]")
    _need(tuple(lv_pool.shape) == lead + (n_pages, r, page), "lv_pool must be [(n_agents,) n_pages, r, page]")
    _need(tuple(b_k.shape) == (n_agents, r, h_kv * d) and b_v.shape == b_k.shape,
          "b_k/b_v must be [n_agents, r, H_kv*d]")
    _need(ctx_req_start.shape == (n_ctx + 1,) and ctx_len.shape == (n_ctx,)
          and req_agent.shape == (n_req,), "index array shapes")
    _need((rope_cos is None) == (rope_sin is None), "rope_cos and rope_sin go together")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _contig(name, t)
            _need(t.dtype == torch.float32 and t.shape[0] >= max(max_ctx_len, 1)
                  and t.shape[1] == d // 2, f"{name} must be fp32 [>=max_ctx_len, d/2]")
    if out is None:
        out = torch.empty_like(q)
    _contig("out", out)
    dims = _dims(h_q, h_kv, d, r, dt, softmax_scale, lr_stride)
    ws_bytes = int(lib.lra_attn_decode_workspace_size(ctypes.byref(dims), n_req, n_ctx,
                                                      max_req_per_ctx, max_ctx_len))
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(dims), _ptr(q), n_req, _ptr(ctx_req_start), n_ctx, max_req_per_ctx,
            _ptr(req_agent), _ptr(k_pool), _ptr(v_pool), _ptr(lk_pool), _ptr(lv_pool), n_pages, page,
            _ptr(block_table), max_blocks, _ptr(ctx_len), max_ctx_len, _ptr(b_k), _ptr(b_v), n_agents,
            _ptr(rope_cos), _ptr(rope_sin), _rows(rope_cos), _ptr(out), _ptr(workspace), wsz,
            _stream(q, stream))
    if _prepare:
        keep = (dims, q, ctx_req_start, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table, ctx_len,
                b_k, b_v, rope_cos, rope_sin, out, workspace)
        return PreparedCall(lib.lra_attn_decode, args, keep, out)
    _check(lib.lra_attn_decode(*args))
    return out


class PreparedCall:
    """One C-ABI call with its arguments checked and marshalled once (``prepare_decode``).
    Calling it issues the same launch again on the same buffers and stream; it holds
    references to every tensor it points into.  ``out`` is the output tensor."""

    def __init__(self, fn, args, keep, out):
        self._fn, self._args, self._keep, self.out = fn, args, keep, out

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _check(st)
        return self.out


def prepare_decode(*args, **kwargs):
    """``decode`` with its validation and argument marshalling done once: returns a
    PreparedCall whose every call launches the decode on the same tensors (whose contents
    may change between calls) and stream.  For loops that call the decode on fixed
    buffers, such as one serving step after another."""
    return decode(*args, _prepare=True, **kwargs)


def decode_noalloc(q, ctx_req_start, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table,
                   ctx_len, b_k, b_v, out, *, max_req_per_ctx, max_ctx_len, rope_cos=None,
                   rope_sin=None, softmax_scale=0.0, stream=None):
    """Decode that allocates nothing (``lra_attn_decode_noalloc``): the arguments of
    ``decode`` without a workspace; ``out`` [n_req, H_q, d] must be given.  The split-K
    scratch is the library's own per-GPU array, so calls that overlap on one GPU race."""
    import torch
    lib = load()
    n_req, h_q, d = q.shape
    n_pages, h_kv, d8, page, eight = k_pool.shape
    _need(d8 * 8 == d and eight == 8, "k_pool must be [n_pages, H_kv, d/8, page, 8]")
    r = lk_pool.shape[-1]
    n_ctx, max_blocks = block_table.shape
    n_agents = b_k.shape[0]
    per_agent = lk_pool.dim() == 4
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("lk_pool", lk_pool),
                    ("lv_pool", lv_pool), ("b_k", b_k), ("b_v", b_v), ("out", out)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from q")
    for name, t in (("ctx_req_start", ctx_req_start), ("req_agent", req_agent),
                    ("block_table", block_table), ("ctx_len", ctx_len)):
        _contig(name, t)
        _need(t.dtype == torch.int32, f"{name} must be int32")
    _need(tuple(out.shape) == tuple(q.shape), "out must be [n_req, H_q, d]")
    lead = (n_agents,) if per_agent else ()
    _need(tuple(v_pool.shape) == (n_pages, h_kv, d, page), "v_pool must be [n_pages, H_kv, d, page]")
    _need(tuple(lk_pool.shape) == lead + (n_pages, page, r), "lk_pool must be [(n_agents,) n_pages, page, r]")
    _need(tuple(lv_pool.shape) == lead + (n_pages, r, page), "lv_pool must be [(n_agents,) n_pages, r, page]")
    _need((rope_cos is None) == (rope_sin is None), "rope_cos and rope_sin go together")
    dims = _dims(h_q, h_kv, d, r, dt, softmax_scale, n_pages * page * r if per_agent else 0)
    _check(lib.lra_attn_decode_noalloc(
        ctypes.byref(dims), _ptr(q), n_req, _ptr(ctx_req_start), n_ctx, max_req_per_ctx,
        _ptr(req_agent), _ptr(k_pool), _ptr(v_pool), _ptr(lk_pool), _ptr(lv_pool), n_pages, page,
        _ptr(block_table), max_blocks, _ptr(ctx_len), max_ctx_len, _ptr(b_k), _ptr(b_v), n_agents,
        _ptr(rope_cos), _ptr(rope_sin), _rows(rope_cos), _ptr(out), _stream(q, stream)))
    return out


def prefill(q, req_agent, k_base, v_base, l_k, l_v, b_k, b_v, *, rope_cos=None, rope_sin=None,
            out=None, softmax_scale=0.0, stream=None, _prepare=False):
    """Chunked prefill (``lra_attn_prefill``): q [n_req, q_len, H_q, d] over
    k_base/v_base [H_kv, kv_len, d], l_k/l_v [kv_len, r] (shared) or [n_agents, kv_len, r]
    (one LR cache per agent); optional RoPE tables [kv_len, d/2] fp32 rotate the adapter
    key term."""
    import torch
    lib = load()
    n_req, q_len, h_q, d = q.shape
    h_kv, kv_len, _ = k_base.shape
    r = l_k.shape[-1]
    n_agents = b_k.shape[0]
    per_agent = l_k.dim() == 3
    lead = (n_agents,) if per_agent else ()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k_base", k_base), ("v_base", v_base), ("l_k", l_k), ("l_v", l_v),
                    ("b_k", b_k), ("b_v", b_v)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from q")
    _contig("req_agent", req_agent)
    _need(req_agent.dtype == torch.int32 and req_agent.shape == (n_req,), "req_agent [n_req] int32")
    _need(tuple(v_base.shape) == (h_kv, kv_len, d), "v_base shape")
    _need(tuple(l_k.shape) == lead + (kv_len, r) and tuple(l_v.shape) == lead + (kv_len, r),
          "l_k/l_v [(n_agents,) kv_len, r]")
    _need(tuple(b_k.shape) == (n_agents, r, h_kv * d) and b_v.shape == b_k.shape, "b_k/b_v shape")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _contig(name, t)
            _need(t.dtype == torch.float32 and t.shape[0] >= kv_len and t.shape[1] == d // 2,
                  f"{name} must be fp32 [>=kv_len, d/2]")
    if out is None:
        out = torch.empty_like(q)
    _contig("out", out)
    dims = _dims(h_q, h_kv, d, r, dt, softmax_scale, kv_len * r if per_agent else 0)
    args = (ctypes.byref(dims), _ptr(q), n_req, q_len, _ptr(req_agent), _ptr(k_base), _ptr(v_base),
            kv_len, _ptr(l_k), _ptr(l_v), _ptr(b_k), _ptr(b_v), n_agents, _ptr(rope_cos),
            _ptr(rope_sin), _rows(rope_cos), _ptr(out), _stream(q, stream))
    if _prepare:
        keep = (dims, q, req_agent, k_base, v_base, l_k, l_v, b_k, b_v, rope_cos, rope_sin, out)
        return PreparedCall(lib.lra_attn_prefill, args, keep, out)
    _check(lib.lra_attn_prefill(*args))
    return out


def prepare_prefill(*args, **kwargs):
    """``prefill`` with its validation and argument marshalling done once (a PreparedCall,
    as ``prepare_decode``)."""
    return prefill(*args, _prepare=True, **kwargs)


def lr_cache_build_workspace_size(*, dtype, n_tok, d_model, rank, n_lr=1):
    """Workspace bytes of ``lra_lr_cache_build`` for these sizes (0: none used)."""
    return int(load().lra_lr_cache_build_workspace_size(dtype, n_tok, d_model, rank, n_lr))


def lr_cache_build(x, a_k, a_v, l_k, l_v, *, row_offset=0, workspace=None, split=True, stream=None):
    """LR-cache rows ``L[row_offset + i] = x[i] A`` (``lra_lr_cache_build``).

    x [n_tok, d_model]; a_k, a_v [r, d_model] (LoRA A weight layout, out x in) and
    l_k, l_v [>= row_offset + n_tok, r], written in place; or, one A per agent,
    a_k, a_v [n_agents, r, d_model] and l_k, l_v [n_agents, rows, r] (X [A_1 .. A_n]).
    ``workspace`` (uint8, zero-filled before first use) is allocated when the split
    build needs one and none is given; ``split=False`` passes none (single-pass kernel).
    """
    lib = load()
    n_tok, d_model = x.shape
    r = a_k.shape[-2]
    n_lr = a_k.shape[0] if a_k.dim() == 3 else 1
    dt = _dtype_code(x)
    for name, t in (("x", x), ("a_k", a_k), ("a_v", a_v), ("l_k", l_k), ("l_v", l_v)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from x")
    lead = (n_lr,) if a_k.dim() == 3 else ()
    _need(tuple(a_k.shape) == lead + (r, d_model) and tuple(a_v.shape) == lead + (r, d_model),
          "a_k/a_v [(n_lr,) r, d_model]")
    _need(l_k.dim() == len(lead) + 2 and l_k.shape[-1] == r and l_v.shape == l_k.shape
          and tuple(l_k.shape[:len(lead)]) == lead, "l_k/l_v [(n_lr,) rows, r]")
    rows = l_k.shape[-2]
    _need(rows >= row_offset + n_tok, "l_k/l_v too short for row_offset + n_tok")
    if not split:
        workspace = None
    elif workspace is None:
        import torch
        n_ws = int(lib.lra_lr_cache_build_workspace_size(dt, n_tok, d_model, r, n_lr))
        if n_ws > 0:
            workspace = torch.zeros(n_ws, dtype=torch.uint8, device=x.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lra_lr_cache_build(dt, _ptr(x), n_tok, d_model, _ptr(a_k), _ptr(a_v), r, n_lr,
                                  _ptr(l_k), _ptr(l_v), int(row_offset), rows * r if n_lr > 1 else 0,
                                  _ptr(workspace), wsz, _stream(x, stream)))
    return l_k, l_v


def rope_table(theta, head_dim, n_pos, device="cuda", stream=None):
    """fp32 cos/sin tables [n_pos, head_dim/2] of pos * theta^(-2i/d), built on the GPU."""
    import torch
    lib = load()
    cos = torch.empty((n_pos, head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(lib.lra_rope_table_build(float(theta), head_dim, n_pos, _ptr(cos), _ptr(sin),
                                    _stream(cos, stream)))
    return cos, sin


def naive_decode(q, ctx_req_start, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table,
                 ctx_len, b_k, b_v, *, max_req_per_ctx, max_ctx_len, scratch=None,
                 softmax_scale=0.0, stream=None):
    """Measurement baseline (not the method): ``lra_naive_expand_pages`` writes each
    request's K_base + L_k B_k and V_base + L_v B_v to pages of its own, then
    ``lra_attn_decode`` runs plain attention over them (one context per request,
    B = 0).  ``scratch`` (a dict, filled on first use and reusable while the shapes
    stay the same) holds those buffers.  Returns the output [n_req, H_q, d]."""
    import torch
    lib = load()
    n_req, h_q, d = q.shape
    n_pages, h_kv = k_pool.shape[:2]
    r = lk_pool.shape[-1]
    n_ctx, max_blocks = block_table.shape
    n_agents = b_k.shape[0]
    per_agent = lk_pool.dim() == 4  # [n_agents, n_pages, 16, r]: one LR pool per agent
    lead = (n_agents,) if per_agent else ()
    _need(tuple(lk_pool.shape) == lead + (n_pages, 16, r), "lk_pool must be [(n_agents,) n_pages, 16, r]")
    _need(tuple(lv_pool.shape) == lead + (n_pages, r, 16), "lv_pool must be [(n_agents,) n_pages, r, 16]")
    out_blocks = max(1, -(-max_ctx_len // 16))
    _need(out_blocks <= max_blocks, "max_ctx_len exceeds the block table")
    sc = scratch if scratch is not None else {}
    if sc.get("key") != (n_req, h_kv, d, r, out_blocks, str(q.dtype)):
        dev = q.device
        sc.clear()
        sc["key"] = (n_req, h_kv, d, r, out_blocks, str(q.dtype))
        sc["k"] = torch.empty((n_req * out_blocks,) + tuple(k_pool.shape[1:]), dtype=q.dtype, device=dev)
        sc["v"] = torch.empty((n_req * out_blocks,) + tuple(v_pool.shape[1:]), dtype=q.dtype, device=dev)
        sc["lk"] = torch.zeros((n_req * out_blocks, 16, r), dtype=q.dtype, device=dev)
        sc["lv"] = torch.zeros((n_req * out_blocks, r, 16), dtype=q.dtype, device=dev)
        sc["bz"] = torch.zeros((1, r, h_kv * d), dtype=q.dtype, device=dev)
        sc["agent0"] = torch.zeros(n_req, dtype=torch.int32, device=dev)
        sc["crs"] = torch.arange(n_req + 1, dtype=torch.int32, device=dev)
        sc["bt"] = torch.arange(n_req * out_blocks, dtype=torch.int32, device=dev).view(n_req, out_blocks)
        req_ctx = torch.searchsorted(ctx_req_start[1:].to(torch.int64),
                                     torch.arange(n_req, device=dev), right=True)
        sc["len"] = ctx_len.to(torch.int64)[req_ctx].to(torch.int32).contiguous()
        sc["out"] = torch.empty_like(q)
        sc["ws"] = None
    dims = _dims(h_q, h_kv, d, r, _dtype_code(q), softmax_scale, n_pages * 16 * r if per_agent else 0)
    _check(lib.lra_naive_expand_pages(
        ctypes.byref(dims), n_req, _ptr(ctx_req_start), n_ctx, _ptr(req_agent), _ptr(k_pool),
        _ptr(v_pool), _ptr(lk_pool), _ptr(lv_pool), n_pages, 16, _ptr(block_table), max_blocks,
        _ptr(ctx_len), _ptr(b_k), _ptr(b_v), n_agents, _ptr(sc["k"]), _ptr(sc["v"]), out_blocks,
        _stream(q, stream)))
    if sc["ws"] is None:
        n_ws = decode_workspace_size(n_q_heads=h_q, n_kv_heads=h_kv, head_dim=d, rank=r,
                                     dtype=_dtype_code(q), n_req=n_req, n_ctx=n_req,
                                     max_req_per_ctx=1, max_ctx_len=max_ctx_len)
        sc["ws"] = torch.zeros(max(n_ws, 16), dtype=torch.uint8, device=q.device)
    return decode(q, sc["crs"], sc["agent0"], sc["k"], sc["v"], sc["lk"], sc["lv"], sc["bt"],
                  sc["len"], sc["bz"], sc["bz"], max_req_per_ctx=1, max_ctx_len=max_ctx_len,
                  out=sc["out"], workspace=sc["ws"], softmax_scale=softmax_scale, stream=stream)


def _paged_prefill_args(q, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table_row, kv_len,
                        b_k, b_v, rope_cos, rope_sin, softmax_scale):
    import torch
    n_req, q_len, h_q, d = q.shape
    n_pages, h_kv, d8, page, eight = k_pool.shape
    _need(d8 * 8 == d and eight == 8 and page == 16, "k_pool must be [n_pages, H_kv, d/8, 16, 8]")
    r = lk_pool.shape[-1]
    n_agents = b_k.shape[0]
    per_agent = lk_pool.dim() == 4
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("lk_pool", lk_pool),
                    ("lv_pool", lv_pool), ("b_k", b_k), ("b_v", b_v)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from q")
    for name, t in (("req_agent", req_agent), ("block_table_row", block_table_row)):
        _contig(name, t)
        _need(t.dtype == torch.int32, f"{name} must be int32")
    _need(tuple(v_pool.shape) == (n_pages, h_kv, d, page), "v_pool must be [n_pages, H_kv, d, 16]")
    lead = (n_agents,) if per_agent else ()
    _need(tuple(lk_pool.shape) == lead + (n_pages, page, r), "lk_pool must be [(n_agents,) n_pages, 16, r]")
    _need(tuple(lv_pool.shape) == lead + (n_pages, r, page), "lv_pool must be [(n_agents,) n_pages, r, 16]")
    _need(req_agent.numel() == n_req, "req_agent must hold n_req entries")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _contig(name, t)
            _need(t.dtype == torch.float32 and t.shape[0] >= kv_len and t.shape[1] == d // 2,
                  f"{name} must be fp32 [>=kv_len, d/2]")
    dims = _dims(h_q, h_kv, d, r, dt, softmax_scale, n_pages * page * r if per_agent else 0)
    return dims, (n_req, q_len, n_pages, n_agents)


def prefill_paged(q, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table_row, kv_len, b_k,
                  b_v, *, rope_cos=None, rope_sin=None, out=None, softmax_scale=0.0, stream=None):
    """Chunked prefill over one context read in place from the paged pools
    (``lra_attn_prefill_paged``): q [n_req, q_len, H_q, d]; pools as in ``decode`` (LR
    pools [n_pages, 16, r] / [n_pages, r, 16], or with a leading n_agents dimension for
    one LR cache per agent); block_table_row [max_blocks] int32.  No workspace."""
    import torch
    lib = load()
    dims, (n_req, q_len, n_pages, n_agents) = _paged_prefill_args(
        q, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table_row, kv_len, b_k, b_v,
        rope_cos, rope_sin, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _contig("out", out)
    _check(lib.lra_attn_prefill_paged(
        ctypes.byref(dims), _ptr(q), n_req, q_len, _ptr(req_agent), _ptr(k_pool), _ptr(v_pool),
        _ptr(lk_pool), _ptr(lv_pool), n_pages, 16, _ptr(block_table_row),
        block_table_row.shape[0], kv_len, _ptr(b_k), _ptr(b_v), n_agents, _ptr(rope_cos),
        _ptr(rope_sin), _rows(rope_cos), _ptr(out), _stream(q, stream)))
    return out


def prefill_paged_staged_workspace_size(*, n_q_heads, n_kv_heads, head_dim, rank, kv_len):
    """Bytes of workspace ``prefill_paged_staged`` needs for a context of ``kv_len`` tokens."""
    dims = _dims(n_q_heads, n_kv_heads, head_dim, rank, LRA_BF16, 0.0)
    return int(load().lra_attn_prefill_paged_staged_workspace_size(ctypes.byref(dims), kv_len))


def prefill_paged_staged(q, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table_row, kv_len,
                         b_k, b_v, *, rope_cos=None, rope_sin=None, out=None, workspace=None,
                         softmax_scale=0.0, stream=None):
    """The paged prefill through a contiguous staging copy (``lra_attn_prefill_paged_staged``);
    arguments as in ``prefill_paged`` (shared LR pools only); ``workspace`` (uint8) is
    allocated when not given."""
    import torch
    lib = load()
    dims, (n_req, q_len, n_pages, n_agents) = _paged_prefill_args(
        q, req_agent, k_pool, v_pool, lk_pool, lv_pool, block_table_row, kv_len, b_k, b_v,
        rope_cos, rope_sin, softmax_scale)
    need = int(lib.lra_attn_prefill_paged_staged_workspace_size(ctypes.byref(dims), kv_len))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _contig("out", out)
    _check(lib.lra_attn_prefill_paged_staged(
        ctypes.byref(dims), _ptr(q), n_req, q_len, _ptr(req_agent), _ptr(k_pool), _ptr(v_pool),
        _ptr(lk_pool), _ptr(lv_pool), n_pages, 16, _ptr(block_table_row),
        block_table_row.shape[0], kv_len, _ptr(b_k), _ptr(b_v), n_agents, _ptr(rope_cos),
        _ptr(rope_sin), _rows(rope_cos), _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(q, stream)))
    return out


def cache_append(slot_mapping, k_new, v_new, lk_new, lv_new, k_pool, v_pool, lk_pool, lv_pool,
                 *, n_q_heads=None, stream=None):
    """Write new tokens' K/V rows [n_tok, H_kv, d] and LR rows [n_tok, r] into the paged
    pools at ``slot_mapping`` [n_tok] int64 (``lra_cache_append``).  With one LR pool per
    agent (lk_pool [n_agents, n_pages, 16, r]) the LR rows are [n_agents, n_tok, r], set a
    going to agent a's pools."""
    import torch
    lib = load()
    n_tok, h_kv, d = k_new.shape
    r = lk_new.shape[-1]
    n_pages = k_pool.shape[0]
    per_agent = lk_pool.dim() == 4
    n_lr = lk_pool.shape[0] if per_agent else 1
    for name, t in (("k_new", k_new), ("v_new", v_new), ("lk_new", lk_new), ("lv_new", lv_new),
                    ("k_pool", k_pool), ("v_pool", v_pool), ("lk_pool", lk_pool),
                    ("lv_pool", lv_pool), ("slot_mapping", slot_mapping)):
        _contig(name, t)
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (n_tok,), "slot_mapping [n_tok] int64")
    lead = (n_lr,) if per_agent else ()
    _need(tuple(v_new.shape) == (n_tok, h_kv, d) and tuple(lk_new.shape) == lead + (n_tok, r)
          and tuple(lv_new.shape) == lead + (n_tok, r), "new row shapes")
    _need(tuple(lk_pool.shape) == lead + (n_pages, 16, r) and tuple(lv_pool.shape) == lead + (n_pages, r, 16),
          "LR pool shapes")
    dims = _dims(n_q_heads or h_kv, h_kv, d, r, _dtype_code(k_new), 0.0, n_pages * 16 * r if per_agent else 0)
    _check(lib.lra_cache_append(ctypes.byref(dims), n_tok, _ptr(slot_mapping), _ptr(k_new),
                                _ptr(v_new), _ptr(lk_new), _ptr(lv_new), n_lr, _ptr(k_pool), _ptr(v_pool),
                                _ptr(lk_pool), _ptr(lv_pool), n_pages, 16, _stream(k_new, stream)))


def naive_prefill_workspace_size(*, n_q_heads, n_kv_heads, head_dim, rank, n_req, kv_len):
    """Bytes of the expanded caches ``naive_prefill`` writes (bf16)."""
    dims = _dims(n_q_heads, n_kv_heads, head_dim, rank, LRA_BF16, 0.0)
    return int(load().lra_naive_prefill_workspace_size(ctypes.byref(dims), n_req, kv_len))


def naive_prefill(q, req_agent, k_base, v_base, l_k, l_v, b_k, b_v, *, rope_cos=None, rope_sin=None,
                  out=None, workspace=None, softmax_scale=0.0, stream=None):
    """Measurement baseline (not the method, ``lra_naive_prefill``): each request's
    K_base + rot(L_k B_k) and V_base + L_v B_v written to ``workspace`` (uint8, allocated
    when not given), then plain causal attention over them.  Arguments as in ``prefill``."""
    import torch
    lib = load()
    n_req, q_len, h_q, d = q.shape
    h_kv, kv_len, _ = k_base.shape
    r = l_k.shape[-1]
    n_agents = b_k.shape[0]
    per_agent = l_k.dim() == 3
    lead = (n_agents,) if per_agent else ()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k_base", k_base), ("v_base", v_base), ("l_k", l_k), ("l_v", l_v),
                    ("b_k", b_k), ("b_v", b_v)):
        _contig(name, t)
        _need(_dtype_code(t) == dt, f"{name} dtype differs from q")
    _contig("req_agent", req_agent)
    _need(req_agent.dtype == torch.int32 and req_agent.shape == (n_req,), "req_agent [n_req] int32")
    _need(tuple(v_base.shape) == (h_kv, kv_len, d), "v_base shape")
    _need(tuple(l_k.shape) == lead + (kv_len, r) and tuple(l_v.shape) == lead + (kv_len, r),
          "l_k/l_v [(n_agents,) kv_len, r]")
    _need(tuple(b_k.shape) == (n_agents, r, h_kv * d) and b_v.shape == b_k.shape, "b_k/b_v shape")
    if rope_cos is not None:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _contig(name, t)
            _need(t.dtype == torch.float32 and t.shape[0] >= kv_len and t.shape[1] == d // 2,
                  f"{name} must be fp32 [>=kv_len, d/2]")
    if out is None:
        out = torch.empty_like(q)
    _contig("out", out)
    dims = _dims(h_q, h_kv, d, r, dt, softmax_scale, kv_len * r if per_agent else 0)
    need = int(lib.lra_naive_prefill_workspace_size(ctypes.byref(dims), n_req, kv_len))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.lra_naive_prefill(
        ctypes.byref(dims), _ptr(q), n_req, q_len, _ptr(req_agent), _ptr(k_base), _ptr(v_base),
        kv_len, _ptr(l_k), _ptr(l_v), _ptr(b_k), _ptr(b_v), n_agents, _ptr(rope_cos),
        _ptr(rope_sin), _rows(rope_cos), _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(q, stream)))
    return out


def ceiling_hbm_read(buf, sink, *, n_workgroups=0, nontemporal=True, chunked=False, stream=None):
    """Device ceiling, not part of the method: ``lra_ceiling_hbm_read`` streams every
    byte of the contiguous device tensor ``buf`` (its size a multiple of 16 bytes)
    and keeps nothing; ``sink`` is a small device tensor (>= 4 bytes).  ``chunked``:
    each workgroup reads one contiguous chunk, else a grid-stride sweep."""
    lib = load()
    _contig("buf", buf)
    flags = (1 if nontemporal else 0) | (2 if chunked else 0)
    _check(lib.lra_ceiling_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), int(n_workgroups), flags,
                                    _ptr(sink), _stream(buf, stream)))


def ceiling_mfma_bf16(sink, *, n_workgroups, iters, lds_operands=0, stream=None):
    """Device ceiling, not part of the method: ``lra_ceiling_mfma_bf16`` issues
    n_workgroups * iters * 524288 flops of bf16 MFMA, ``lds_operands`` (0, 1 or 2)
    of each MFMA's operands read from LDS.  Returns that flop count."""
    lib = load()
    _check(lib.lra_ceiling_mfma_bf16(int(lds_operands), int(n_workgroups), int(iters), _ptr(sink),
                                     _stream(sink, stream)))
    return int(n_workgroups) * int(iters) * 524288
