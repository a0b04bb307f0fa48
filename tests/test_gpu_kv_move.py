"""Device KV-row moves (mla_kv_commit, mla_kv_defrag) against the CPU oracle,
bit for bit, and the attention's result before and after a move."""
import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import inputs as I
from oracle import kv_move as K

pytestmark = pytest.mark.gpu


def rand_pool(P, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 1 << 16, (P, 576), generator=g, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_commit(pool, table, seq, N, lens, paths, base):
    gp, gt = pool.cuda(), table.cuda()
    M.kv_commit(gp, gt, torch.tensor(seq, dtype=torch.int32).cuda(), N,
                torch.tensor(lens, dtype=torch.int32).cuda(),
                torch.tensor(np.asarray(paths), dtype=torch.int32).cuda(),
                torch.tensor(base, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    return bits(gp), gt.cpu().numpy()


def test_commit_hand_example_and_swap():
    pool = rand_pool(16, 1)
    table = torch.tensor([[0, 1, 2, 3, 4, 5, 12, 9, 14, 7]], dtype=torch.int32)
    gp, gt = run_commit(pool, table, [10], 4, [2], [[0, 2, 0, 0]], [0])
    ep, et = K.kv_commit(bits(pool), table.numpy(), [10], 4, [2], [[0, 2, 0, 0]], [0])
    assert np.array_equal(gp, ep) and np.array_equal(gt, et)
    table = torch.tensor([[0, 1, 2, 3, 7, 6]], dtype=torch.int32)
    gp, gt = run_commit(pool, table, [6], 2, [2], [[0, 1]], [2])  # destinations = crossed sources
    ep, et = K.kv_commit(bits(pool), table.numpy(), [6], 2, [2], [[0, 1]], [2])
    assert np.array_equal(gp, ep) and np.array_equal(gt, et)


def root_path(parents, v):
    path = []
    while v >= 0:
        path.append(v)
        v = parents[v]
    return path[::-1]


@pytest.mark.parametrize("n", [8, 16, 64])
@pytest.mark.parametrize("in_place", [False, True])
def test_random_commits_bit_exact(n, in_place):
    rng = np.random.default_rng(100 + n + in_place)
    B, P, max_kv = 8, 32768, 1200
    pool = rand_pool(P, n)
    table = np.zeros((B, max_kv), dtype=np.int32)
    seq, lens, paths, base = [], [], np.zeros((B, n), dtype=np.int32), []
    free = rng.permutation(P // 2)  # scattered source slots in the lower half
    for b in range(B):
        S = int(rng.integers(n, max_kv + 1))
        rb = P // 2 + b * max_kv  # the request's run in the upper half
        table[b, :S] = free[b * max_kv: b * max_kv + S]
        if in_place:  # tree nodes allocated inside the run, in node order
            table[b, S - n:S] = rb + (S - n) + np.arange(n)
        par = I.random_parents(n, 8, 7 + b)
        path = root_path(par, int(rng.integers(0, n)))
        paths[b, :len(path)] = path
        seq.append(S)
        lens.append(len(path) if b % 3 else int(rng.integers(0, len(path) + 1)))
        base.append(rb)
    gp, gt = run_commit(pool, torch.from_numpy(table), seq, n, lens, paths, base)
    ep, et = K.kv_commit(bits(pool), table, seq, n, lens, paths, base)
    assert np.array_equal(gt, et)
    assert np.array_equal(gp, ep)


def test_defrag_bit_exact():
    rng = np.random.default_rng(3)
    B, P, max_kv = 3, 65536, 13000
    pool = rand_pool(P, 11)
    seq = [5000, 0, 12345]
    table = rng.permutation(B * max_kv).reshape(B, max_kv).astype(np.int32)
    base = [40000, 46000, 51000]
    gp, gt = pool.cuda(), torch.from_numpy(table).cuda()
    M.kv_defrag(gp, gt, torch.tensor(seq, dtype=torch.int32).cuda(), torch.tensor(base, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    ep, et = K.kv_defrag(bits(pool), table, seq, base)
    assert np.array_equal(gt.cpu().numpy(), et)
    assert np.array_equal(bits(gp), ep)


def test_defrag_short_rows_and_runs_past_the_pool():
    """Tables shorter than one 32-row pass (a pass spans several sequences),
    many passes per workgroup, out-of-range table entries (clamped reads) and
    runs that end past the pool (those rows are skipped and their table
    entries kept)."""
    rng = np.random.default_rng(5)
    B, P, max_kv = 3000, 40000, 7
    pool = rand_pool(P, 12)
    seq = [int(x) for x in rng.integers(0, max_kv + 1, size=B)]
    table = rng.integers(0, P // 2, size=(B, max_kv)).astype(np.int32)
    table[rng.random((B, max_kv)) < 0.01] = -5          # clamped to slot 0
    table[rng.random((B, max_kv)) < 0.01] = P + 123     # clamped to the last slot
    # disjoint runs of 8 slots in the upper half, so no run holds a source: the
    # clamped slot P - 1 would be position 7 of a run (never a row), and the
    # last runs end past the pool
    base = [P // 2 + 8 * b for b in range(B)]
    assert base[-1] + max_kv > P and (P - 1 - P // 2) % 8 >= max_kv
    gp, gt = pool.cuda(), torch.from_numpy(table).cuda()
    M.kv_defrag(gp, gt, torch.tensor(seq, dtype=torch.int32).cuda(), torch.tensor(base, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    ep, et = K.kv_defrag(bits(pool), table, seq, base)
    assert np.array_equal(gt.cpu().numpy(), et)
    assert np.array_equal(bits(gp), ep)


def test_defrag_at_189k_keeps_rows_and_attention():
    wl = I.config_workload(3, device="cuda", ctx=189440)
    before = [t.clone() for t in M.verify_workload(wl)]
    S = wl.seq_lens_host()[0]
    P = wl.num_slots
    # a fresh run in a larger pool: the old pool's rows stay where they were
    pool = torch.empty((P + S, 576), dtype=torch.bfloat16, device="cuda")
    pool[:P] = wl.kv_pool
    old_table = wl.page_table.clone()
    M.kv_defrag(pool, wl.page_table, wl.seq_lens, torch.tensor([P], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(wl.page_table[0, :S], P + torch.arange(S, dtype=torch.int32, device="cuda"))
    assert torch.equal(pool.view(torch.int16)[P:P + S], wl.kv_pool.view(torch.int16)[old_table[0, :S].long()])
    wl.kv_pool = pool
    after = M.verify_workload(wl)
    assert torch.equal(after[0].view(torch.int16), before[0].view(torch.int16))
    assert torch.equal(after[1].view(torch.int32), before[1].view(torch.int32))
