"""Pins of the KV-move oracle (oracle/kv_move.py): hand-worked cases and the
invariants a move must keep."""
import numpy as np

from oracle import kv_move as K


def pool_of(P, seed=0):
    """P distinct rows of 576 16-bit patterns (row r starts with r)."""
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 1 << 16, size=(P, 576), dtype=np.uint16)
    pool[:, 0] = np.arange(P, dtype=np.uint16)
    return pool


def test_commit_hand_example():
    P, N = 16, 4
    pool = pool_of(P)
    table = np.array([[0, 1, 2, 3, 4, 5, 12, 9, 14, 7]], dtype=np.int32)  # S = 10, tree at 6..9
    new_pool, new_table = K.kv_commit(pool, table, [10], N, [2], [[0, 2, 0, 0]], [0])
    # accepted nodes 0 and 2 (slots 12 and 14) land at slots 6 and 7
    assert np.array_equal(new_table, [[0, 1, 2, 3, 4, 5, 6, 7, 14, 7]])
    assert np.array_equal(new_pool[6], pool[12]) and np.array_equal(new_pool[7], pool[14])
    untouched = [r for r in range(P) if r not in (6, 7)]
    assert np.array_equal(new_pool[untouched], pool[untouched])


def test_commit_reads_before_writing_a_swap():
    P, N = 12, 2
    pool = pool_of(P, 1)
    table = np.array([[0, 1, 2, 3, 7, 6]], dtype=np.int32)  # S = 6, nodes at slots 7, 6
    new_pool, new_table = K.kv_commit(pool, table, [6], N, [2], [[0, 1]], [0])
    assert np.array_equal(new_pool[4], pool[7]) and np.array_equal(new_pool[5], pool[6])
    # base = 2: destinations 6 and 7 are exactly the sources, crossed
    new_pool, new_table = K.kv_commit(pool, table, [6], N, [2], [[0, 1]], [2])
    assert np.array_equal(new_pool[6], pool[7]) and np.array_equal(new_pool[7], pool[6])
    assert np.array_equal(new_table, [[0, 1, 2, 3, 6, 7]])


def test_commit_keeps_logical_content_and_clamps():
    rng = np.random.default_rng(5)
    P, N, B, max_kv = 4096, 16, 4, 600
    pool = pool_of(P, 2)
    table = rng.permutation(B * max_kv).reshape(B, max_kv).astype(np.int32)  # sources below 2400
    seq = [500, 17, 600, 16]
    lens = [3, 16, 0, 99]          # 99 clamps to N
    paths = rng.integers(-3, 20, size=(B, N))  # out-of-range nodes clamp
    base = [2048, 2600, 3200, 3700]
    new_pool, new_table = K.kv_commit(pool, table, seq, N, lens, paths, base)
    for b in range(B):
        S = min(max(seq[b], N), max_kv)
        t0, L = S - N, min(max(lens[b], 0), N)
        for k in range(L):
            n = min(max(paths[b, k], 0), N - 1)
            assert new_table[b, t0 + k] == base[b] + t0 + k
            assert np.array_equal(new_pool[new_table[b, t0 + k]], pool[table[b, t0 + n]])
        assert np.array_equal(new_table[b, :t0], table[b, :t0])
        assert np.array_equal(new_table[b, t0 + L:], table[b, t0 + L:])


def test_defrag_moves_every_row_and_rewrites_the_table():
    rng = np.random.default_rng(9)
    P, B, max_kv = 3000, 3, 500
    pool = pool_of(P, 3)
    table = rng.permutation(1500).reshape(B, max_kv).astype(np.int32)
    seq = [500, 0, 321]
    base = [1500, 2000, 2600]
    new_pool, new_table = K.kv_defrag(pool, table, seq, base)
    dest = set()
    for b in range(B):
        S = seq[b]
        assert np.array_equal(new_table[b, :S], base[b] + np.arange(S))
        assert np.array_equal(new_table[b, S:], table[b, S:])
        assert np.array_equal(new_pool[new_table[b, :S]], pool[table[b, :S]])  # same logical rows
        dest.update(range(base[b], base[b] + S))
    untouched = [r for r in range(P) if r not in dest]
    assert np.array_equal(new_pool[untouched], pool[untouched])


def test_defrag_is_idempotent_on_a_contiguous_sequence():
    P = 100
    pool = pool_of(P, 4)
    table = (40 + np.arange(30, dtype=np.int32)).reshape(1, 30)
    new_pool, new_table = K.kv_defrag(pool, table, [30], [40])
    assert np.array_equal(new_pool, pool) and np.array_equal(new_table, table)
