"""The token index of a route, r // K, as the kernels compute it: a multiply-high by
kinv = floor(2^32 / K) + 1.

The unit-table builds (moe_group, moe_plan_group and the one-launch grouped form) take a
route's token with this product instead of an integer division.  kinv exceeds 2^32 / K
by less than 1, so r * kinv / 2^32 exceeds r / K by less than r / 2^32 < 2^-16, which is
below 1 / K for K <= 64: the floor never moves.  Checked here for every route index the
boundary admits (B * topk <= 65536) and every topk 1..64.
"""
import numpy as np


def test_multiply_high_token_index_is_exact():
    r = np.arange(65536, dtype=np.uint64)
    for K in range(1, 65):
        kinv = np.uint64((1 << 32) // K + 1)
        got = (r * kinv) >> np.uint64(32)
        np.testing.assert_array_equal(got, r // np.uint64(K), err_msg=f"K={K}")


def test_plain_truncated_reciprocal_would_not_be():
    # without the + 1 the product falls short at the multiples of K (r = K gives 0)
    r = np.arange(1, 65536, dtype=np.uint64)
    K = 3
    kinv = np.uint64((1 << 32) // K)
    assert np.any(((r * kinv) >> np.uint64(32)) != r // np.uint64(K))
