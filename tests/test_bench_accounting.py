"""The benchmark's algorithmic byte/flop accounting against closed forms (CPU)."""
import numpy as np

import bench


def test_decode_bytes_shared_contexts():
    # 4 contexts x 8192 tokens, 16 requests, 4 agents, Hq32 Hkv8 d128 r16, bf16:
    # caches 4*8192*(2*8*128 + 2*16)*2 = 136,314,880; Q and O 131,072 each;
    # B 4 agents * 2 * 16 * 1024 * 2 = 262,144; index arrays 8,292.
    got = bench.decode_bytes([8192] * 4, 16, 4, 32, 8, 128, 16)
    assert got == 136_314_880 + 131_072 * 2 + 262_144 + 2048 * 4 + 16 + 20 + 64


def test_sharing_ratio_matches_page_closed_form():
    # Non-Shared: N agents each stream a private cache; BaseLRShared: one base cache and one
    # rank-r LR cache for all N.  Per token and per side (K or V): N*d_out vs d_out + r, i.e.
    # the ratio 1/N + r/(N d_out) of LRAgent §3.  The benchmark's unshared count is N private
    # copies of the shared stream, so shared/unshared = 1/N exactly.
    n, r, d_out = 4, 16, 8 * 128
    shared = bench.decode_bytes([8192], 4, 4, 32, 8, 128, 16) - (4 * 32 * 128 * 2 * 2 + 4 * 2 * 16 * 1024 * 2
                                                                + 512 * 4 + 4 + 8 + 16)
    unshared_private_lr = n * 8192 * 2 * (d_out + r) * 2
    assert shared * n == unshared_private_lr
    value_side = (8192 * d_out + 8192 * r) / (n * 8192 * d_out)
    assert abs(value_side - (1 / n + r / (n * d_out))) < 1e-15
    assert bench.decode_bytes_unshared([8192] * 4, 32, 8, 128, 16) == n * shared


def test_prefill_flops_closed_forms():
    # 512 new over 16384, 4 agents, RoPE: 5.957e11 (rebuild at head dim, per-row B_v)
    f = bench.prefill_flops(4, 512, 16896, 32, 8, 128, 16, rope=True)
    pairs = 512 * 16384 + 512 * 513 // 2
    assert pairs == 8_519_936
    assert f == 4 * 32 * pairs * (512 + 32) + 4 * 512 * 32 * 2 * 16 * 128 + 16896 * 8 * 4 * 2 * 16 * 128
    assert abs(f / 5.957e11 - 1) < 1e-3
    # one (agent, layer) of the 4096-over-131072 step without RoPE: 32 heads x pairs x 576
    f5 = bench.prefill_flops(1, 4096, 135168, 32, 8, 128, 16, rope=False)
    pairs5 = 4096 * 131072 + 4096 * 4097 // 2
    assert pairs5 == 545_261_568
    assert f5 == 32 * pairs5 * 576 + 4096 * 32 * 2 * 16 * 128 * 2


def test_lr_build_bytes():
    assert bench.lr_build_bytes(4096, 4096, 16) == (4096 * 4096 + 2 * 16 * 4096 + 2 * 4096 * 16) * 2


def test_committed_counter_summary_is_of_the_current_kernel_sources():
    """profiles/hbm_traffic__all_legs.txt was taken on the kernel sources in the tree, and
    every HBM- or MFMA-bound leg bench.py reports (and the read ceilings) has its record, so
    the bench's `roofline.traffic` is measured, not null.  A kernel change without a new
    profiling session fails here."""
    import bench
    legs = ("primary", "decode_rope", "decode_qkvo_r4", "decode_per_agent", "naive_decode", "paged_decode",
            "naive_paged_decode", "prefill_rope", "prefill_paged", "naive_prefill", "lr_build", "prelr_step",
            "ceilings", "ceilings_read_hbm_read_chunked_kernel<true>", "ceilings_read_hbm_read_kernel<true>")
    for leg in legs:
        traffic, src = bench.measured_traffic(leg)
        assert traffic is not None, f"{leg}: {src}"
        assert traffic > 0 and "rocprofv3" in src
    # the read ceiling moves what it reads: 1 GiB per launch within the counters' granularity
    assert abs(bench.measured_traffic("ceilings_read_hbm_read_chunked_kernel<true>")[0] - (1 << 30)) < (1 << 20)
    # the decode's measured traffic is within 10% of its algorithmic bytes (no wasted re-reads)
    alg = bench.decode_bytes([8192] * 4, 16, 4, 32, 8, 128, 16)
    assert 1.0 <= bench.measured_traffic("primary")[0] / alg < 1.1
