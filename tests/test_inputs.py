"""Seeded input generators: determinism and the structure each config asks for."""
import numpy as np
import torch

from mla_tree_verify_02_amd import inputs as I


def test_same_seed_same_bytes():
    a = I.config_workload(1)
    b = I.config_workload(1)
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.kv_pool.view(torch.int16), b.kv_pool.view(torch.int16))
    assert torch.equal(a.page_table, b.page_table)
    assert torch.equal(a.tree_mask, b.tree_mask)
    c = I.config_workload(1, layer=1)
    assert not torch.equal(a.q.view(torch.int16), c.q.view(torch.int16))


def test_seed_formula():
    assert I.seed_for(3, 7, I.F_Q) == 3_007_001


def test_chain_mask_is_lower_triangular_with_diagonal():
    m = I.ancestor_bitmask(I.chain_parents(8))
    assert [int(x) for x in m[:, 0]] == [(1 << (i + 1)) - 1 for i in range(8)]


def test_heap_binary_tree_shape():
    p = I.heap_binary_parents(16)
    d = I.tree_depths(p)
    assert d.max() == 4 and d[15] == 4 and list(p[:4]) == [-1, 0, 0, 1]


def test_random_tree_constraints():
    p = I.random_parents(64, 8, seed=123)
    d = I.tree_depths(p)
    assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 64))
    assert d.max() <= 8
    m = I.ancestor_bitmask(p)
    assert m.shape == (64, 2)
    for i in range(64):
        bits = [(int(m[i, j // 32]) >> (j % 32)) & 1 for j in range(64)]
        assert sum(bits) == d[i] + 1          # itself and each ancestor once
        assert bits[i] == 1 and all(b == 0 for b in bits[i + 1:])


def test_scattered_table_is_injective_and_disjoint():
    wl = I.make_workload(batch=3, num_nodes=4, num_heads=1, prefix_lens=[50, 7, 90],
                         num_slots=512, config_id=7)
    t = wl.np_page_table()
    seen = np.concatenate([t[b, :s] for b, s in enumerate(wl.np_seq_lens())])
    assert len(np.unique(seen)) == len(seen)
    assert seen.min() >= 0 and seen.max() < 512


def test_runs64_layout():
    wl = I.make_workload(batch=2, num_nodes=8, num_heads=1, prefix_lens=[200, 70],
                         num_slots=4096, layout="runs64", config_id=8)
    t = wl.np_page_table()
    for b, s in enumerate(wl.np_seq_lens()):
        row = t[b, :s].astype(np.int64)
        for k in range(0, s, 64):
            run = row[k:k + 64]
            assert run[0] % 64 == 0 and np.array_equal(run, run[0] + np.arange(len(run)))


def test_unreferenced_slots_are_nan():
    wl = I.make_workload(batch=1, num_nodes=2, num_heads=1, prefix_lens=[10], num_slots=64,
                         config_id=9)
    used = set(wl.np_page_table()[0, :12].tolist())
    kv = wl.kv_pool.float()
    for s in range(64):
        assert bool(torch.isnan(kv[s]).all()) == (s not in used)


def test_config_shapes():
    wl = I.config_workload(1)
    assert tuple(wl.q.shape) == (1, 8, 8, 576) and wl.max_kv == 1032 and wl.num_slots == 4096
    pre = I.log_uniform_prefixes(8, 1024, 131072, I.seed_for(5, 0, I.F_LENS))
    assert all(1024 <= p <= 131072 for p in pre)


def test_relayout_moves_every_referenced_row_and_nothing_else():
    wl = I.make_workload(batch=2, num_nodes=8, num_heads=2, prefix_lens=[300, 77],
                         num_slots=1024, tree="binary", config_id=7)
    for seed, layout in [(5, "scattered"), (6, "runs64")]:
        other = I.relayout(wl, seed, layout)
        old = wl.kv_pool.view(torch.int16)
        new = other.kv_pool.view(torch.int16)
        referenced = torch.zeros(wl.num_slots, dtype=torch.bool)
        for b, s in enumerate(wl.seq_lens_host()):
            t_old, t_new = wl.page_table[b, :s].long(), other.page_table[b, :s].long()
            assert torch.equal(new[t_new], old[t_old])
            referenced[t_new] = True
        assert bool((new[~referenced] == I.BF16_NAN_BITS).all())
        assert torch.equal(other.q, wl.q) and np.array_equal(other.np_mask(), wl.np_mask())
        assert other.seq_lens_host() == wl.seq_lens_host() and other.scale == wl.scale
