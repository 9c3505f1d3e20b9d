"""Host-side arithmetic of bench.py (no GPU): the algorithmic byte counts
against plain enumerations of the cycles."""
import numpy as np

import bench
from refs import pass_list


def test_sym_pass_bytes_matches_enumeration():
    for (n, bw, tw, es) in [(40, 8, 3, 8), (33, 5, 4, 4), (100, 16, 15, 4), (64, 2, 1, 8)]:
        for (b, t) in pass_list(bw, tw):
            total = 0
            for R in range(max(n - (b - t) - 1, 0)):
                k = 0
                while R + (b - t) + k * b <= n - 2:
                    c = R + (b - t) + k * b
                    ch = min(c + t, n - 1)
                    m = ch - c + 1
                    p = R if k == 0 else c - b
                    entries = m                      # pivot row segment
                    entries += (c - p - 1) * m       # rows above the block
                    entries += m * (m + 1) // 2      # the block's upper triangle
                    entries += (min(ch + b, n - 1) - ch) * m  # columns to the right
                    total += 2 * es * entries
                    k += 1
            assert bench.sym_pass_bytes(n, b, t, es) == total


def test_memory_level_by_working_set():
    import bench
    assert bench.memory_level(1 << 20) == "l2"
    assert bench.memory_level(8651520) == "infinity_cache"  # the n = 16384, BW = 64 fp32 working band
    assert bench.memory_level(300 << 20) == "hbm"


def test_cycle_kernel_names():
    import bench
    assert bench.is_cycle_kernel("void bb::(anonymous namespace)::k_group<float, 17, 100, false>(float*, int)", "f32")
    assert not bench.is_cycle_kernel("void bb::(anonymous namespace)::k_group<float, 17, 0, true>(float*, int)", "f32")
    assert bench.is_cycle_kernel("void bb::(anonymous namespace)::k_persist<double, 33, 16>(double*, long)", "f64")
    assert bench.is_cycle_kernel("void bb::(anonymous namespace)::k_persist<double, 33, 16, true>(double*, long)", "f64")
    assert bench.is_cycle_kernel("void bb::(anonymous namespace)::k_persist<float, 32, 16, false>(float*, long)", "f32")
    assert not bench.is_cycle_kernel("void bb::(anonymous namespace)::k_persist<float, 32, 16, true>(float*)", "f64")
    assert not bench.is_cycle_kernel("bb::(anonymous namespace)::k_probe_stream(float const*, long, int)", "f32")
