"""The algorithmic bytes bench.py divides by the step time, against the
closed forms of the step: per layer, the attention projections
(2*d*H*hd + 2*d*G*hd weights), the router (d*E), the union of routed experts
plus the shared expert (3*d*F each) and the K and V rows read (2*G*hd per
position and sequence), all bf16."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.workloads import ATTN92_B1, MOE16_B1, TINY  # noqa: E402


def test_attn92_batch1_step_bytes():
    w = ATTN92_B1
    b_e = 3 * 4096 * 1024 * 2
    assert b_e == 25_165_824
    attn = (2 * 4096 * 32 * 128 + 2 * 4096 * 8 * 128) * 2
    assert attn == 83_886_080
    kv = 2 * 8 * 128 * 4096 * 2  # K and V rows of 4096 past positions
    per_layer = attn + 9 * b_e + 4096 * 64 * 2 + kv
    assert per_layer == 327_680_000
    weights = bench.step_bytes(w, 1, 1, [8] * 92, 0)
    assert weights + 92 * kv == 92 * per_layer == 30_146_560_000


def test_moe16_batch1_step_bytes():
    w = MOE16_B1
    b_e = 3 * 2048 * 1024 * 2
    assert b_e == 12_582_912
    per_layer = 7 * b_e + 2048 * 64 * 2
    assert per_layer == 88_342_528
    assert bench.step_bytes(w, 1, 1, [6] * 16, 0) == 16 * per_layer == 1_413_480_448


def test_union_and_fp32_accounting():
    # batch 8: each union expert counts once per layer, the shared expert once
    w = MOE16_B1.with_(M=8)
    b_e = 3 * 2048 * 1024 * 2
    unions = [29, 31, 26, 30]
    got = bench.step_bytes(w.with_(L=4), 8, 8, unions, 0)
    assert got == sum((u + 1) * b_e + 2048 * 64 * 2 for u in unions)
    # the fp32 stack: 4-byte weights, no shared expert, no attention
    assert bench.step_bytes(TINY, 1, 1, [2, 2], 0) == 2 * (2 * 3 * 256 * 512 * 4 + 256 * 8 * 4)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: asked for more, it exits with status 2 and a
    message, before touching a device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""
