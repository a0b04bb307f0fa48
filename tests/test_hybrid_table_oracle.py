"""Pins of the hybrid-paging expansion (oracle/hybrid_table.py) and of the
hybrid-layout input generator."""
import numpy as np
import torch

from mla_tree_verify_02_amd import inputs as I
from oracle import hybrid_table as H


def test_hand_example():
    pages = np.array([[5, 2, 9]])
    tree = np.array([[100, 7, 33]])
    t = H.expand(pages, tree, [13], 3, 4, 16)  # prefix of 10: pages 5, 2, 9 (partial)
    assert list(t[0]) == [20, 21, 22, 23, 8, 9, 10, 11, 36, 37, 100, 7, 33, 0, 0, 0]


def test_page_size_one_is_the_page_list():
    rng = np.random.default_rng(0)
    pages = rng.permutation(1000)[:50].reshape(2, 25)
    tree = rng.integers(0, 1000, size=(2, 4))
    t = H.expand(pages, tree, [29, 12], 4, 1, 40)
    assert np.array_equal(t[0, :25], pages[0]) and np.array_equal(t[0, 25:29], tree[0])
    assert np.array_equal(t[1, :8], pages[1, :8]) and np.array_equal(t[1, 8:12], tree[1])


def test_consecutive_pages_are_the_identity():
    t = H.expand(np.arange(10).reshape(1, 10), np.array([[640, 641]]), [642], 2, 64, 700)
    assert np.array_equal(t[0, :640], np.arange(640)) and list(t[0, 640:642]) == [640, 641]


def test_page_beyond_the_row_reads_the_last_entry():
    t = H.expand(np.array([[3, 8]]), np.array([[1]]), [14], 1, 4, 16)  # prefix 13 > 2 pages
    assert list(t[0, 8:13]) == [32, 33, 34, 35, 32]


def test_generator_agrees_with_the_expansion_and_keeps_rows():
    wl = I.make_workload(batch=3, num_nodes=8, num_heads=2, prefix_lens=[500, 64, 3],
                         num_slots=4096, tree="binary", config_id=11)
    hl = I.hybrid_layout(wl, 64, 5)
    seq = wl.seq_lens_host()
    t = H.expand(hl.prefix_pages.numpy(), hl.tree_slots.numpy(), seq, 8, 64, wl.max_kv)
    for b, s in enumerate(seq):
        assert np.array_equal(t[b, :s], hl.workload.page_table[b, :s].numpy())
        new = hl.workload.kv_pool.view(torch.int16)[hl.workload.page_table[b, :s].long()]
        old = wl.kv_pool.view(torch.int16)[wl.page_table[b, :s].long()]
        assert torch.equal(new, old)
    # tree rows sit outside every prefix page
    pages = set(int(x) for b, s in enumerate(seq) for x in hl.prefix_pages[b, :(s - 8 + 63) // 64])
    assert all(int(x) // 64 not in pages for x in hl.tree_slots.flatten())
