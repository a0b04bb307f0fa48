"""Pins of the input-check oracle: hand-built inputs whose out-of-range counts
are known by construction."""
import numpy as np
import pytest

from oracle.input_check import check_inputs


def valid_case(B=3, N=8, max_kv=40, P=100, seed=0):
    rng = np.random.default_rng(seed)
    sl = rng.integers(N, max_kv + 1, size=B).astype(np.int32)
    pt = rng.integers(0, P, size=(B, max_kv)).astype(np.int32)
    W = (N + 31) // 32
    mk = np.zeros((B, N, W), dtype=np.uint32)
    for i in range(N):
        mk[:, i, i // 32] |= np.uint32(1 << (i % 32))
    return pt, sl, mk


def test_valid_inputs_count_nothing():
    pt, sl, mk = valid_case()
    assert check_inputs(pt, sl, mk, 8, 100) == [0, 0, 0]


def test_lengths_outside_range_and_their_clamp():
    N, max_kv, P = 4, 10, 50
    pt = np.zeros((3, max_kv), dtype=np.int32)
    sl = np.array([2, 12, 7], dtype=np.int32)  # below N, above max_kv, fine
    mk = np.ones((3, N, 1), dtype=np.uint32)
    # table entries: bad ones only count below the clamped length (4, 10, 7)
    pt[0, 3] = -1    # p < 4: counts
    pt[0, 4] = P     # p >= 4: not read
    pt[1, 9] = P     # p < 10: counts
    pt[2, 6] = 10 ** 9  # p < 7: counts
    pt[2, 7] = -5    # p >= 7: not read
    assert check_inputs(pt, sl, mk, N, P) == [2, 3, 0]


def test_slot_bounds_are_half_open():
    pt = np.array([[0, 49, 50, -1]], dtype=np.int32)
    sl = np.array([4], dtype=np.int32)
    mk = np.ones((1, 2, 1), dtype=np.uint32)
    assert check_inputs(pt, sl, mk, 2, 50) == [0, 2, 0]


@pytest.mark.parametrize("N,bits,expect", [
    (5, [(0, 4)], 0),           # node 4 is the last node
    (5, [(0, 5)], 1),           # node 5 does not exist
    (5, [(0, 31)], 1),
    (32, [(0, 31)], 0),         # a full word: no spare bits
    (33, [(1, 0)], 0),          # node 32, second word
    (33, [(1, 1)], 1),          # node 33 does not exist
    (64, [(1, 31)], 0),
    (40, [(0, 3), (1, 8), (1, 2)], 1),  # several bits in one row: one row counted
])
def test_mask_bits_past_the_last_node(N, bits, expect):
    W = (N + 31) // 32
    mk = np.zeros((1, N, W), dtype=np.uint32)
    for w, b in bits:
        mk[0, N - 1, w] |= np.uint32(1 << b)
    pt = np.zeros((1, N), dtype=np.int32)
    sl = np.array([N], dtype=np.int32)
    assert check_inputs(pt, sl, mk, N, 1) == [0, 0, expect]


def test_counts_add_over_planted_faults():
    """Random valid inputs with faults planted at known places: three table
    faults per sequence below its length, junk past every length, two bad
    lengths whose clamped values cover the same positions, three mask rows."""
    rng = np.random.default_rng(7)
    B, N, max_kv, P = 6, 40, 300, 1000
    pt, sl, mk = valid_case(B, N, max_kv, P, seed=7)
    sl[:] = np.clip(sl, N + 10, max_kv)
    sl[2] = N       # becomes N - 1 below: clamped back to N
    sl[4] = max_kv  # becomes max_kv + 1 below: clamped back to max_kv
    for b in range(B):
        for p in rng.choice(int(sl[b]), size=3, replace=False):
            pt[b, p] = rng.choice([-1, P, P + 12345, -(1 << 30)])
        pt[b, int(sl[b]):] = -1  # past the end: never counted
    for b, i in [(1, 0), (3, 39), (5, 17)]:
        mk[b, i, 1] |= np.uint32(1 << 9)  # node 41 of 40
    sl[2] = N - 1
    sl[4] = max_kv + 1
    assert check_inputs(pt, sl, mk, N, P) == [2, 3 * B, 3]
