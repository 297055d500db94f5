"""bench.py's own arithmetic and contract, without a GPU: the algorithmic
byte counts it divides by (the attend's per-call bytes against the table of
bytes per (sequence, kv head) the long-context attend moves, the flush's
bytes per element), its statistics helper, and the refusal of a multi-GPU
run."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flush_bytes_per_element():
    # 2 B fp16 in, bits/8 B of codes, 8 B of binary32 scale and zero per 32
    assert bench.algo_bytes_per_elem(4) == 2.75
    assert bench.algo_bytes_per_elem(2) == 2.5
    assert bench.algo_bytes_per_elem(4, True) == 4.75
    # the full cache: 1.208e9 elements per tensor, 3.322 GB per 4-bit launch
    assert 288 * 32768 * 128 * bench.algo_bytes_per_elem(4) == 3321888768


def test_flush_bytes_at_other_head_dims():
    # head_dim 128: the per-element figure for keys and values alike
    for keys in (True, False):
        assert bench.flush_bytes(288, 32768, 128, 4, keys) == 3321888768
    # head_dim 80, 2 slabs x 64 tokens: 10240 elements, 2 B in and 0.5 B of
    # codes each; keys 2 token groups x 80 channels x 2 slabs = 320 pairs,
    # values 3 groups (32, 32, 16 channels) x 128 tokens = 384 pairs
    assert bench.flush_bytes(2, 64, 80, 4, True) == 10240 * 2.5 + 320 * 8
    assert bench.flush_bytes(2, 64, 80, 4, False) == 10240 * 2.5 + 384 * 8
    # a ragged last key group still costs one pair per channel
    assert bench.flush_bytes(1, 33, 16, 2, True) == 33 * 16 * 2 + 33 * 16 // 4 + 2 * 16 * 8


def test_attend_bytes_per_call():
    # per (sequence, kv head): S_kv x 192 B of 4-bit codes and binary32
    # metadata at head_dim 128, plus 128 residual tokens x 512 B
    for B, S, mb in ((1, 2048, 3.67), (4, 2048, 14.7), (16, 2048, 58.7), (32, 2048, 117.4),
                     (1, 16384, 25.7), (4, 16384, 102.8), (16, 16384, 411.0), (32, 16384, 822.1)):
        got = bench.attend_bytes(B * 8, S, 128, 4)
        assert got == B * 8 * (S * 192 + 128 * 512)
        assert abs(got / 1e6 - mb) < 0.06, (B, S, got)
    # binary16 scale/zero: 160 B per stored token and kv head
    assert bench.attend_bytes(1, 1, 0, 4, pair_bytes=4) == 160
    # groups of 64 / 128: the codes' 128 B plus one 8-byte scale/zero pair per
    # channel per group of keys and per group of a token's values: 160 / 144 B
    assert bench.attend_bytes(1, 1, 0, 4, group=64) == 160
    assert bench.attend_bytes(1, 1, 0, 4, group=128) == 144
    # head_dim 256: twice the codes and metadata
    assert bench.attend_bytes(1, 1, 0, 4, head_dim=256) == 384
    # head_dim 80: 2 x 40 B of codes, 20 B of key metadata per token, and
    # three value groups (32, 32 and 16 channels) of 8 B
    assert bench.attend_bytes(1, 1, 0, 4, head_dim=80) == 124


def test_stats_are_order_statistics():
    s = bench.stats([3.0, 1.0, 2.0, 5.0, 4.0])
    assert s == {"min": 1.0, "median": 3.0, "max": 5.0, "n": 5}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
