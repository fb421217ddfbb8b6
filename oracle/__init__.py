"""CPU oracle for Flash-LoRA-Attention — TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(``attention_shared_base_amd``) never imports it, and this package imports
nothing from the product.  The two share no code; the only shared module is
``workloads`` (seeded synthetic inputs, which contains none of the method's
arithmetic).

What it computes, in plain float64 NumPy (``reference.py``) and in plain
Python loops for tiny shapes (``brute.py``):

* the materialised definition of multi-LoRA attention over a shared base
  cache plus a shared low-rank (LR) cache, ``softmax(Q K^T * scale) V`` with
  ``K = K_base + rot(L_k B_k)`` and ``V = V_base + L_v B_v``
  (LRAgent, arXiv 2602.01053v2 — App. A.3 cache decomposition
  ``Y = X W0 + X A B``; §3 BaseShared/BaseLRShared; App. D.1 for the key-side
  adapter and the RoPE rotation);
* the reordered Flash-LoRA form ``P V_base + (P V_lr) B`` and the augmented
  head-dimension form, used only to pin the identities the pages state
  (§3 "Flash-LoRA-Attention", App. B);
* the LR-cache build ``L = X A`` (PReCache abstract: the shared context's
  hidden states are multiplied by the adapters' input matrices when first
  processed; LRAgent §3 BaseLRShared with shared A);
* rotate-half RoPE tables in float64.

Pins (``tests/test_oracle_*.py``, CPU only): brute-force loops, ``B = 0``
reducing to plain attention (checked against torch's SDPA on CPU in float64),
the reordered/materialised identity and the RoPE barrier, softmax rows summing
to one, closed-form special cases and the hand-derived fixtures in
``tests/golden/``.
"""
from .reference import (  # noqa: F401
    causal_visible,
    rope_inv_freq,
    rope_tables,
    rope_rotate_half,
    attention_materialised,
    attention_reordered,
    attention_augmented,
    gather_pages,
    decode_paged,
    prefill,
    lr_cache_build,
    softmax_two_pass,
)
