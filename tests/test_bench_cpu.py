"""Host-side checks of the benchmark: its refusal of more than one GPU and the
algorithmic counts it divides by."""
import os
import subprocess
import sys

from mla_latent_decode_amd.inputs import DSV3, TINY
from mla_latent_decode_amd.layout import (append_bytes_per_token, cache_bytes_per_token,
                                          decode_flops_per_token, train_attention_flops)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cache_bytes_match_the_layout():
    assert cache_bytes_per_token(DSV3, True) == 1184      # 1024 + 128 + 8 * 4
    assert cache_bytes_per_token(DSV3, False) == 1152
    assert cache_bytes_per_token(TINY, True) == 4 * (32 + 8) + 4 * 2
    assert append_bytes_per_token(DSV3) == 2 * (512 + 64) + 1184
    assert decode_flops_per_token(DSV3) == 2 * 128 * (512 + 64) + 2 * 128 * 512


def test_training_flops_count_every_causal_pair():
    B, T = 2, 5
    pairs = sum(1 for b in range(B) for h in range(DSV3.n_heads) for i in range(T)
                for j in range(i + 1))
    f, bwd = train_attention_flops(DSV3, B, T)
    assert f == 2 * pairs * (192 + 128)
    assert bwd == 2 * pairs * (3 * 192 + 2 * 128)
