"""Seeded synthetic tensors and storage-format helpers.

Shared by the tests, the benchmark and the oracle's callers.  Holds none of the
method's arithmetic: only random draws, rounding to the storage type, and
layout moves (paging) of data that already exists.

Random streams.  Every tensor is drawn from its own PCG64 stream keyed by
``SeedSequence(entropy=seed, spawn_key=(tag, layer, chunk))`` in chunks of
``CHUNK`` values, so the values do not depend on draw order or on the number of
threads used to fill them.  Normal draws are float32 ``standard_normal`` scaled
by ``sigma`` in float32, then (for bf16 storage) rounded once to bfloat16 by
round-to-nearest-even.  Both the GPU and the oracle read those exact bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 20

# Stream tags: one per logical tensor kind.
TAG_Q, TAG_K, TAG_V, TAG_LK, TAG_LV, TAG_BK, TAG_BV = 1, 2, 3, 4, 5, 6, 7
TAG_X, TAG_AK, TAG_AV, TAG_QDEC, TAG_PERM, TAG_LEN = 8, 9, 10, 11, 12, 13


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(n):
    return [(i, i * CHUNK, min(n, (i + 1) * CHUNK)) for i in range((n + CHUNK - 1) // CHUNK)]


def normal_f32(seed, tag, shape, sigma=1.0, layer=0):
    """float32 N(0, sigma^2) array of ``shape`` from stream ``(seed, tag, layer)``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    sig = np.float32(sigma)

    def fill(c):
        i, a, b = c
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag, layer, i))
        rng = np.random.Generator(np.random.PCG64(ss))
        rng.standard_normal(out=out[a:b], dtype=np.float32)
        if sig != 1:
            out[a:b] *= sig

    ch = _chunks(n)
    if len(ch) <= 2:
        for c in ch:
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, ch))
    return out.reshape(shape)


def rng_for(seed, tag, layer=0):
    """A single PCG64 generator for small integer draws (lengths, permutations)."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=(tag, layer, 0))))


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Inputs here are finite draws, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def conv(c):
        _, a, b = c
        u = flat[a:b].view(np.uint32)
        out[a:b] = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
                    >> np.uint32(16)).astype(np.uint16)

    ch = _chunks(flat.size)
    if len(ch) <= 2:
        for c in ch:
            conv(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(conv, ch))
    return out.reshape(x.shape)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bits (uint16) exactly to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a):
    """Exact float64 view of stored values: uint16 arrays are bf16 bits, floats pass through."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def draw(seed, tag, shape, sigma, dtype, layer=0):
    """Normal draw stored as ``dtype`` ('f32' -> float32, 'bf16' -> uint16 bits)."""
    x = normal_f32(seed, tag, shape, sigma, layer)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def paginate(kv, lr, page_ids, n_pages, page):
    """Scatter one context's contiguous caches into page pools.

    ``kv`` ``[H_kv, L, d]`` -> pool ``[n_pages, H_kv, page, d]``; ``lr``
    ``[L, r]`` -> pool ``[n_pages, page, r]``; logical page ``b`` goes to pool
    page ``page_ids[b]``.  Slots past ``L`` in the last page are zero.
    """
    h_kv, length, d = kv.shape
    r = lr.shape[1]
    kvp = np.zeros((n_pages, h_kv, page, d), dtype=kv.dtype)
    lrp = np.zeros((n_pages, page, r), dtype=lr.dtype)
    for blk in range((length + page - 1) // page):
        t0 = blk * page
        n = min(page, length - t0)
        kvp[page_ids[blk], :, :n, :] = kv[:, t0:t0 + n, :]
        lrp[page_ids[blk], :n, :] = lr[t0:t0 + n, :]
    return kvp, lrp


def decode_device_layout(k_pool, v_pool, lk_pool, lv_pool):
    """Reorder logical page pools into the decode kernel's page layouts.

    Logical: K, V ``[n_pages, H_kv, page, d]``; L_k, L_v ``[n_pages, page, r]``.
    Device:  K ``[n_pages, H_kv, d/8, page, 8]``, V ``[n_pages, H_kv, d, page]``,
             L_k ``[n_pages, page, r]``, L_v ``[n_pages, r, page]``.
    Pure data movement (same values, different order).
    """
    n_pages, h_kv, page, d = k_pool.shape
    k = np.ascontiguousarray(k_pool.reshape(n_pages, h_kv, page, d // 8, 8).transpose(0, 1, 3, 2, 4))
    v = np.ascontiguousarray(v_pool.transpose(0, 1, 3, 2))
    lk = np.ascontiguousarray(lk_pool)
    lv = np.ascontiguousarray(lv_pool.transpose(0, 2, 1))
    return k, v, lk, lv
