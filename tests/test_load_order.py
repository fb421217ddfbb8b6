"""The binding loads torch's HIP runtime before the library, whatever the caller
imported first: a fresh interpreter that loads the library without importing torch
itself ends up with exactly one libamdhip64 mapped."""
import os
import subprocess
import sys

import pytest

import attention_shared_base_amd as lra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(lra.lib_path),
                                reason="liblra_attn.so not built (run __graft_entry__.build())")


def test_one_hip_runtime_when_the_library_is_loaded_first():
    code = ("import attention_shared_base_amd as lra; lra.load(); import torch; "
            "maps = open('/proc/self/maps').read().splitlines(); "
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"
