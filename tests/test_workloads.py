"""Seeded input generators: reproducibility, bf16 rounding, paging layout (CPU)."""
import numpy as np
import pytest

import workloads as w
from workloads import synth


def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        # exact ties: low 16 bits 0x8000 with even/odd kept bit
                        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF],
                                 dtype=np.uint32).view(np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_deterministic_and_chunk_independent():
    a = synth.normal_f32(9, 1, (3 * synth.CHUNK + 17,))
    b = synth.normal_f32(9, 1, (3 * synth.CHUNK + 17,))
    assert np.array_equal(a, b)
    c = synth.normal_f32(9, 2, (1000,))
    assert not np.array_equal(a[:1000], c)
    # a prefix of a larger draw equals the smaller draw (chunked streams)
    d = synth.normal_f32(9, 1, (1000,))
    assert np.array_equal(a[:1000], d)


def test_config_shapes():
    dec, pre = w.config1()
    assert dec.q.shape == (2, 4, 64) and dec.q.dtype == np.float32
    assert pre.q.shape == (2, 16, 4, 64) and pre.kv_len == 256
    assert list(dec.ctx_req_start()) == [0, 2]
    c2 = w.config2()
    assert c2.k_pool.shape == (2048, 8, 16, 128) and c2.k_pool.dtype == np.uint16
    assert list(c2.req_ctx) == [b // 4 for b in range(16)]
    assert list(c2.req_agent) == [b % 4 for b in range(16)]
    lens = w.config4_lengths()
    assert lens.min() >= 4096 and lens.max() <= 65536 and len(lens) == 32


def test_shuffled_table_is_a_permutation():
    c = w.make_decode(3, dtype="bf16", ctx_lens=[40, 17, 64], reqs=[(0, 0), (1, 1), (2, 0)],
                      n_agents=2, h_q=4, h_kv=2, d=8, r=4, shuffle=True)
    used = np.concatenate([c.block_table[i, :(int(n) + 15) // 16] for i, n in enumerate(c.ctx_len)])
    assert sorted(used.tolist()) == list(range(c.k_pool.shape[0]))
