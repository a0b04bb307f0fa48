"""GPU parity of the split kernel's two-row-block form.

Calls with at least 16 row groups of 64 query rows whose slices hold at least
48 tiles, or at least 8 row groups with slices of at least 64 tiles, run two
row groups per workgroup (two 16-row blocks per wave). The
plan is recognised by its slice count; tolerances and the comparison are those
of test_gpu_parity (out 2e-2 abs + rel, lse 1e-3 abs + rel, in fp32).
"""
import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import inputs as I

from test_gpu_parity import compare, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def slicing(batch, rows, max_kv, rb):
    """Slices per sequence and tiles per slice of a plan with rb row groups per
    workgroup: G = ceil(CUs / workgroup groups) slots, c = ceil(B T / G') for
    T tiles per sequence (G' = G - (B - 1) when that is more than half of G)."""
    groups = -(-(-(-rows // 64)) // rb)
    slots = max(1, -(-cus() // groups))
    tiles = -(-max_kv // 32)
    target = slots - (batch - 1) if slots > 2 * (batch - 1) else slots
    c = min(-(-(batch * tiles) // target), tiles)
    return -(-tiles // c), c


def assert_two_row_blocks(wl):
    rows = wl.num_nodes * wl.num_heads
    plan = M.plan_query(M.make_shape(wl.batch, wl.num_nodes, wl.num_heads, wl.max_kv, wl.num_slots), cus())
    splits, c = slicing(wl.batch, rows, wl.max_kv, 2)
    assert (rows >= 16 * 64 and c >= 48) or (rows >= 8 * 64 and c >= 64), (rows, c)
    assert plan["splits"] == splits and plan["chunk"] == 32 * c, (plan, splits, c)


def rows_of_every_group(wl, per_group, seed):
    """per_group rows from every 64-row group of every sequence, plus the
    first and last row."""
    R = wl.num_nodes * wl.num_heads
    rng = np.random.default_rng(seed)
    pick = [0, wl.batch * R - 1]
    for b in range(wl.batch):
        for g0 in range(0, R, 64):
            n = min(64, R - g0)
            pick.extend(b * R + g0 + rng.choice(n, size=min(per_group, n), replace=False))
    return np.unique(pick)


@pytest.mark.parametrize("q_gain", [1.0, 4.0])
def test_odd_number_of_row_groups(oracle_mod, q_gain):
    """64 nodes x 17 heads: 17 row groups, so the last workgroup group holds
    one row group (its second row block reads no Q and stores nothing)."""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=17, prefix_lens=[131072], num_slots=262144,
                         tree="random", max_depth=8, config_id=120, device="cuda", q_gain=q_gain)
    assert_two_row_blocks(wl)
    compare(wl, oracle_mod, rows=rows_of_every_group(wl, 2, seed=120),
            label=f"two row blocks, 17 row groups gain{q_gain}")


def test_late_score_jump_raises_the_reference_mid_slice(oracle_mod):
    """Keys from position 63000 on are scaled by 4 (exact in bf16), so the
    slice holding that position meets scores far above its first tile's:
    some rows raise their reference mid-slice and O is rescaled."""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=16, prefix_lens=[131072], num_slots=262144,
                         tree="random", max_depth=8, config_id=121, device="cuda")
    assert_two_row_blocks(wl)
    splits, c = slicing(1, 64 * 16, wl.max_kv, 2)
    assert (63000 // 32) % c > 8, "the jump must fall inside a slice, not at its start"
    slots = wl.page_table[0, 63000:wl.seq_lens_host()[0]].long()
    wl.kv_pool[slots] = wl.kv_pool[slots] * 4
    compare(wl, oracle_mod, rows=rows_of_every_group(wl, 2, seed=121), label="two row blocks, late jump")


def test_batch_of_two(oracle_mod):
    """Two sequences of 64 x 16 rows (131000 and 70000 keys): the batch
    slicing with two row groups per workgroup."""
    wl = I.make_workload(batch=2, num_nodes=64, num_heads=16, prefix_lens=[131000, 70000],
                         num_slots=262144, tree="random", max_depth=8, config_id=122, device="cuda",
                         q_gain=4.0)
    assert_two_row_blocks(wl)
    compare(wl, oracle_mod, rows=rows_of_every_group(wl, 1, seed=122), label="two row blocks, batch 2")


def test_short_sequence_ignores_stale_workspace(oracle_mod):
    """One sequence of 9000 keys under a plan for 131136: the slices past the
    sequence write the empty partial for both row groups of their
    workgroup, over a workspace of NaN bytes."""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=16, prefix_lens=[9000], num_slots=65536,
                         tree="random", max_depth=8, config_id=123, device="cuda", max_kv=131136,
                         q_gain=4.0)
    assert_two_row_blocks(wl)
    shape = M.make_shape(1, 64, 16, wl.max_kv, wl.num_slots)
    ws = torch.full((M.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    out, lse = M.verify_workload(wl, workspace=ws)
    torch.cuda.synchronize()
    compare(wl, oracle_mod, rows=rows_of_every_group(wl, 1, seed=123), label="two row blocks, short sequence",
            gpu=(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()))


@pytest.mark.parametrize("cid", [2, 4])
def test_split_then_combine_equals_the_call(cid):
    """mla_tree_verify_splitkv then mla_tree_verify_combine give the bits of
    mla_tree_verify, with one row group per workgroup (binary16-ctx65536) and
    with two (random64-h64-ctx131072)."""
    wl = I.config_workload(cid, device="cuda")
    ref = run_gpu(wl)
    call = M.prepare_workload(wl)
    call.out.zero_()
    call.lse.zero_()
    call.splitkv()
    call.combine()
    torch.cuda.synchronize()
    assert np.array_equal(call.out.view(torch.int16).cpu().numpy().view(np.uint16), ref[0])
    assert np.array_equal(call.lse.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))


@pytest.mark.parametrize("heads,keys", [(16, 49152), (16, 65536), (8, 131072)])
def test_slices_near_the_threshold(oracle_mod, heads, keys):
    """64 nodes x 16 heads at 49,152 and 65,536 keys (49- and 65-tile slices)
    and 64 x 8 at 131,072 (65-tile slices): the shortest slices the
    two-row-group form takes, at gain 4."""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=heads, prefix_lens=[keys], num_slots=262144,
                         tree="random", max_depth=8, config_id=125, device="cuda", q_gain=4.0)
    assert_two_row_blocks(wl)
    compare(wl, oracle_mod, rows=rows_of_every_group(wl, 1, seed=125),
            label=f"two row blocks, 64x{heads} at {keys} keys")


def test_batch_above_64_sequences(oracle_mod):
    """80 sequences of 64 x 16 rows (4,200-6,000 keys each, one slice of at
    least 131 tiles per sequence): more sequences than a wave has lanes, so the
    block-wide slicing path feeds the two-row-group form."""
    rng = np.random.default_rng(124)
    pre = [int(x) for x in rng.integers(4200, 6000, size=80)]
    wl = I.make_workload(batch=80, num_nodes=64, num_heads=16, prefix_lens=pre, num_slots=524288,
                         tree="random", max_depth=8, config_id=124, device="cuda", q_gain=4.0)
    assert_two_row_blocks(wl)
    R = 64 * 16
    rows = np.unique(np.r_[0, 80 * R - 1, [b * R + g * 64 + rng.integers(64)
                                             for b in (0, 1, 37, 63, 64, 79) for g in range(16)]])
    compare(wl, oracle_mod, rows=rows, label="two row blocks, batch 80")


def test_graph_capture_replays_match_eager():
    """A captured two-row-group call (64 x 64 heads at 131072 keys): every
    replay, with eager work between replays, gives the eager call's bits."""
    wl = I.config_workload(4, device="cuda")
    ref = run_gpu(wl)
    call = M.prepare_workload(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run()
    other = I.config_workload(1, device="cuda")
    for _ in range(3):
        call.out.zero_()
        call.lse.zero_()
        g.replay()
        M.verify_workload(other)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(call.out.view(torch.int16).cpu().numpy().view(np.uint16), ref[0])
        assert np.array_equal(call.lse.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))
