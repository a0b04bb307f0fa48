"""mla_tree_verify_noalloc (the entry point whose workspace is the library's
fixed per-GPU scratch) against mla_tree_verify with a caller workspace, both
through the C ABI.

Both run the same kernels on the same inputs, so the outputs must agree bit
for bit. Two calls in a row share the scratch, the second on a smaller
problem, so that stale contents of the first call are in the scratch when the
second one runs.
"""
import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import _lib
from mla_tree_verify_02_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load()


def bits(out, lse):
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()


def with_workspace(wl):
    return bits(*M.verify_workload(wl))


def noalloc(wl):
    out = torch.full((wl.batch, wl.num_nodes, wl.num_heads, 512), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((wl.batch, wl.num_nodes, wl.num_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    M.mla_tree_verify_noalloc(wl.q, wl.kv_pool, wl.page_table, wl.seq_lens, wl.tree_mask, wl.scale,
                              out, lse)
    return bits(out, lse)


def same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_two_calls_second_smaller_single_sequence():
    big = I.config_workload(2, device="cuda", q_gain=4.0)     # 16 nodes x 8 heads, ctx 65536
    small = I.config_workload(1, device="cuda", q_gain=4.0)   # 8 x 8, ctx 1024
    print("noalloc: binary16-ctx65536 then chain8-ctx1024", flush=True)
    assert same(noalloc(big), with_workspace(big))
    assert same(noalloc(small), with_workspace(small))


def test_two_calls_second_smaller_batch():
    big = I.make_workload(batch=6, num_nodes=16, num_heads=8, prefix_lens=[30000, 5, 7000, 120, 2500, 61000],
                          num_slots=131072, tree="binary", config_id=120, device="cuda", q_gain=4.0)
    small = I.make_workload(batch=3, num_nodes=5, num_heads=3, prefix_lens=[0, 31, 1000], num_slots=4096,
                            tree="random", max_depth=3, config_id=121, device="cuda")
    print("noalloc: batch 6 x (16 x 8) then batch 3 x (5 x 3)", flush=True)
    assert same(noalloc(big), with_workspace(big))
    assert same(noalloc(small), with_workspace(small))


def test_oversized_call_is_rejected_and_enqueues_nothing():
    # 1024 sequences of 16 nodes x 8 heads need more partials than the scratch holds
    B, N, H = 1024, 16, 8
    shape = M.make_shape(B, N, H, 64, 4096)
    assert M.workspace_size(shape) > _lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, N, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((4096, 576), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 64, dtype=torch.int32, device="cuda")
    tm = torch.zeros((B, N, 1), dtype=torch.int32, device="cuda")
    out = torch.full((B, N, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, N, H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(M.MtvError) as e:
        M.mla_tree_verify_noalloc(q, kv, pt, sl, tm, 0.1, out, lse)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())


def test_captured_replays_match_eager():
    wl = I.make_workload(batch=2, num_nodes=16, num_heads=8, prefix_lens=[3000, 9000], num_slots=32768,
                         tree="binary", config_id=122, device="cuda")
    ref = with_workspace(wl)
    out = torch.empty((2, 16, 8, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 16, 8), dtype=torch.float32, device="cuda")
    other = I.config_workload(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.mla_tree_verify_noalloc(wl.q, wl.kv_pool, wl.page_table, wl.seq_lens, wl.tree_mask, wl.scale,
                                  out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.mla_tree_verify_noalloc(wl.q, wl.kv_pool, wl.page_table, wl.seq_lens, wl.tree_mask, wl.scale,
                                  out, lse)
    for _ in range(3):
        out.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert same(bits(out, lse), ref)
        noalloc(other)  # another call on the same scratch between replays
