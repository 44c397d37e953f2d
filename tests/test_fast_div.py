"""The prefill kernel divides workgroup ids by the KV head count, the batch and
8 x the query-group size through a multiplier m and shift s made on the host
(fast_div in exact_io_aware_attn_amd/csrc/fwd_bf16.hip):

    s = ceil(log2 d),  m = floor(2^32 (2^s - d) / d) + 1,
    n / d = (umulhi(n, m) + n) >> s   for 0 <= n < 2^31

(division by an invariant integer through a multiply, Granlund and Montgomery
1994). The same arithmetic is written out here and checked against integer
division: every divisor up to 4096 on edge and random numerators, and every
numerator below 2^20 for the divisors the workloads use."""

import numpy as np


def _fast_div(d):
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((1 << 32) * ((1 << s) - d)) // d + 1
    assert 0 < m < (1 << 32) or d == 1
    return m, s


def _apply(n, m, s):
    n = n.astype(np.uint64)
    hi = (n * np.uint64(m)) >> np.uint64(32)  # n < 2^31, m < 2^32: no overflow
    return ((hi + n) & np.uint64(0xFFFFFFFF)) >> np.uint64(s)


def test_every_divisor_up_to_4096_on_edge_and_random_numerators():
    rng = np.random.default_rng(7)
    top = (1 << 31) - 1
    for d in range(1, 4097):
        m, s = _fast_div(d)
        edge = np.array([0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, top, top - 1, top - d],
                        dtype=np.int64)
        n = np.concatenate([edge[edge >= 0], rng.integers(0, top + 1, 256),
                            rng.integers(0, 64 * d + 1, 256)]).astype(np.uint64)
        np.testing.assert_array_equal(_apply(n, m, s), n // np.uint64(d), err_msg=f"d={d}")


def test_every_numerator_below_2_20_for_workload_divisors():
    n = np.arange(1 << 20, dtype=np.uint64)
    for d in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 96, 128):
        m, s = _fast_div(d)
        np.testing.assert_array_equal(_apply(n, m, s), n // np.uint64(d), err_msg=f"d={d}")
