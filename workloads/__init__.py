"""Seeded synthetic inputs shared by tests, benchmark and oracle callers.

Contains no arithmetic of the method itself: random draws, rounding to the
storage type, and page layout only.
"""
from .synth import (f32_to_bf16_bits, bf16_bits_to_f32, widen, draw, normal_f32,  # noqa: F401
                    paginate, rng_for, decode_device_layout)
from .configs import (DecodeCase, PrefillCase, LRBuildCase, PreLRLayerCase,  # noqa: F401
                      make_decode, decode_subset, make_prefill, page_table, make_lr_build, config1, config2, config3,
                      config4, config4_lengths, config5_layer, PAGE)
