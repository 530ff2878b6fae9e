"""The seeded input generator: Philox4x32-10 known answers and the value
mapping of include/synth.h (host side; the device side is checked against
the host in the GPU tests)."""
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers(syn):
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        assert syn.philox(v[0:4], v[4:6]) == tuple(v[6:10])


def test_normal_mapping_matches_definition(syn):
    """Element i comes from block i/4 with counter (i/4, stream) and key seed;
    Box-Muller on (r0, r1) and (r2, r3); values rounded to binary32."""
    seed, stream = 0x1234_5678_9ABC_DEF0, syn.stream_id(5, syn.K_WQ, 3)
    a = syn.host_normal((10,), syn.F32, seed, stream, 0.5, 2.0)
    for blk in range(3):
        ctr = (blk & 0xFFFFFFFF, blk >> 32, stream & 0xFFFFFFFF, stream >> 32)
        r = syn.philox(ctr, (seed & 0xFFFFFFFF, seed >> 32))
        for p in range(2):
            u1 = (r[2 * p] + 1.0) / 2 ** 32
            u2 = r[2 * p + 1] / 2 ** 32
            rad = math.sqrt(-2 * math.log(u1))
            z = (rad * math.cos(2 * math.pi * u2), rad * math.sin(2 * math.pi * u2))
            for q in range(2):
                i = 4 * blk + 2 * p + q
                if i < 10:
                    assert a[i] == np.float32(0.5 + 2.0 * z[q])


def test_uniform_mapping_and_range(syn):
    a = syn.host_uniform((4096,), syn.F32, 7, 9, 0.9, 1.1)
    assert a.min() >= 0.9 and a.max() <= 1.1
    r = syn.philox((0, 0, 9, 0), (7, 0))
    assert a[0] == np.float32(0.9 + 0.2 * ((r[0] + 0.5) / 2 ** 32))


def test_bf16_is_rounded_binary32(syn):
    f = syn.host_normal((1000,), syn.F32, 3, 4, 0.0, 0.02)
    b = syn.host_normal((1000,), syn.BF16, 3, 4, 0.0, 0.02)
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(b, rne)


def test_streams_independent_and_moments(syn):
    a = syn.host_normal((1 << 16,), syn.F32, 1, syn.stream_id(0, syn.K_WGATE, 0))
    b = syn.host_normal((1 << 16,), syn.F32, 1, syn.stream_id(0, syn.K_WGATE, 1))
    assert abs(a.mean()) < 0.02 and abs(a.std() - 1) < 0.02
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.02
    # prefix property: a shorter fill is a prefix of a longer one
    c = syn.host_normal((1001,), syn.F32, 1, syn.stream_id(0, syn.K_WGATE, 0))
    np.testing.assert_array_equal(c, a[:1001])
