"""Device input check (mtv_check_inputs) against the CPU oracle: counts equal
exactly, on valid workloads, on planted faults, across the grid's strides, and
when the call is replayed from a HIP graph."""
import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import inputs as I
from oracle.input_check import check_inputs as oracle_check

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_check(pt, sl, mk, P):
    counts = M.check_inputs(dev(pt.astype(np.int32)), dev(sl.astype(np.int32)),
                            dev(mk.astype(np.uint32).view(np.int32)), P)
    torch.cuda.synchronize()
    return [int(x) for x in counts.cpu()]


def faulty_case(B, N, max_kv, P, seed, faults=3, bad_lens=(), bad_rows=0):
    """Valid inputs plus `faults` out-of-range table entries per sequence (below
    its length), junk past every length, length faults and mask rows with bits
    past node N - 1 (when N is not a multiple of 32)."""
    rng = np.random.default_rng(seed)
    sl = rng.integers(N, max_kv + 1, size=B)
    pt = rng.integers(0, P, size=(B, max_kv))
    for b in range(B):
        k = min(faults, int(sl[b]))
        for p in rng.choice(int(sl[b]), size=k, replace=False):
            pt[b, p] = rng.choice([-1, P, P + 7, -(1 << 31), (1 << 31) - 1])
        pt[b, int(sl[b]):] = rng.integers(-(1 << 31), 1 << 31, size=max_kv - int(sl[b]))
    W = (N + 31) // 32
    mk = rng.integers(0, 1 << 32, size=(B, N, W), dtype=np.uint64).astype(np.uint32)
    spare = N % 32
    if spare:
        mk[:, :, W - 1] &= np.uint32((1 << spare) - 1)
        for _ in range(bad_rows):
            b, i = int(rng.integers(B)), int(rng.integers(N))
            mk[b, i, W - 1] |= np.uint32(1 << int(rng.integers(spare, 32)))
    for b, v in bad_lens:
        sl[b] = v
    return pt, sl, mk


@pytest.mark.parametrize("cid,kw", [(1, {}), (2, {}), (5, {"layout": "scattered"}),
                                    (5, {"layout": "runs64"})])
def test_valid_workloads_count_nothing(cid, kw):
    wl = I.config_workload(cid, device="cuda", **kw)
    counts = M.check_inputs(wl.page_table, wl.seq_lens, wl.tree_mask, wl.num_slots)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0]


@pytest.mark.parametrize("B,N,max_kv,P", [
    (1, 16, 65552, 262144),   # one long table: many workgroups along positions
    (3, 1, 40, 64),
    (8, 31, 5000, 1 << 20),
    (5, 33, 700, 4096),
    (4, 64, 300, 1000),
    (300, 8, 2000, 65536),    # many sequences, several positions each
    (3000, 5, 40, 512),       # more sequences than workgroup rows: the y stride loops
])
def test_planted_faults_match_oracle(B, N, max_kv, P):
    seed = B * 1000 + N
    # two bad lengths: one clamps up to N, one down to max_kv (so the junk past
    # that sequence's old length is read and counted)
    lens = [(0, N - 1), (B - 1, max_kv + 5)] if B > 1 else []
    pt, sl, mk = faulty_case(B, N, max_kv, P, seed, faults=3, bad_lens=lens, bad_rows=4)
    want = oracle_check(pt, sl, mk, N, P)
    got = gpu_check(pt, sl, mk, P)
    assert got == want
    assert want[0] == len(lens) and want[1] > 0


def test_one_long_sequence_exact_count():
    """A headline-sized table (65,552 positions) with faults at the first, the
    last and scattered positions, and junk past the end."""
    N, max_kv, P = 16, 70000, 262144
    S = 65552
    rng = np.random.default_rng(3)
    pt = rng.integers(0, P, size=(1, max_kv))
    where = [0, S - 1, 255, 256, 40000]
    pt[0, where] = [-1, P, -7, P + 1, -(1 << 31)]
    pt[0, S:] = -1
    sl = np.array([S])
    mk = np.zeros((1, N, 1), dtype=np.uint32)
    mk[0, 5, 0] = 1 << 16  # node 16 of 16
    assert gpu_check(pt, sl, mk, P) == [0, len(where), 1]


def test_counts_are_overwritten_and_graph_replays():
    """The counters are cleared by a kernel inside the call, so a captured call
    replays with fresh counts; the inputs change between replays."""
    B, N, max_kv, P = 4, 9, 500, 2048
    pt, sl, mk = faulty_case(B, N, max_kv, P, 11, faults=2, bad_rows=2)
    t_pt, t_sl, t_mk = dev(pt.astype(np.int32)), dev(sl.astype(np.int32)), \
        dev(mk.astype(np.uint32).view(np.int32))
    counts = torch.full((3,), 12345, dtype=torch.int64, device="cuda")
    M.check_inputs(t_pt, t_sl, t_mk, P, counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == oracle_check(pt, sl, mk, N, P)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.check_inputs(t_pt, t_sl, t_mk, P, counts=counts)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.check_inputs(t_pt, t_sl, t_mk, P, counts=counts)
    torch.cuda.synchronize()
    for r in range(4):
        # change the inputs in place: one more fault per replay
        pt[r % B, 0] = -1 - r
        t_pt.copy_(dev(pt.astype(np.int32)))
        counts.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert counts.cpu().tolist() == oracle_check(pt, sl, mk, N, P), r
