"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance (elementwise, compared in fp32): out |g - o| <= 2e-2 + 2e-2 |o|;
lse |g - o| <= 1e-3 + 1e-3 |o|. Page-index and mask handling are checked bit
for bit: a relayout of the same logical rows, poisoned rows that a node may not
see and junk past the sequence end must leave the output bits unchanged.
At long context N(0,1) outputs shrink towards the absolute tolerance, so every
long case also runs a "peaked" variant (Q x 4, exact in bf16) with O(0.1-1)
outputs.
"""
import math
import os

import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import inputs as I

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load()  # raises if the HIP library was not built


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def run_gpu(wl):
    out, lse = M.verify_workload(wl)
    torch.cuda.synchronize()
    return (out.view(torch.int16).cpu().numpy().view(np.uint16),
            lse.cpu().numpy())


def compare(wl, oracle_mod, rows=None, label="", gpu=None):
    """Run both sides (or take the GPU's (out bits, lse) from `gpu`); compare
    all rows or the given flat row ids."""
    g_out, g_lse = run_gpu(wl) if gpu is None else gpu
    o_out, o_lse = oracle_mod.run_workload(wl, rows=rows)
    g_out = bf16_bits_to_f32(g_out).reshape(-1, 512)
    o_out = bf16_bits_to_f32(o_out).reshape(-1, 512)
    g_lse = g_lse.reshape(-1)
    o_lse = o_lse.reshape(-1)
    sel = np.arange(g_lse.size) if rows is None else np.asarray(rows)
    go, oo = g_out[sel].astype(np.float64), o_out[sel].astype(np.float64)
    gl, ol = g_lse[sel].astype(np.float64), o_lse[sel].astype(np.float64)
    assert np.isfinite(go).all(), f"{label}: non-finite GPU output"
    err_o = np.abs(go - oo)
    err_l = np.where(np.isinf(ol) & np.isinf(gl) & (np.sign(ol) == np.sign(gl)), 0.0, np.abs(gl - ol))
    rel_fro = float(np.linalg.norm(go - oo) / max(np.linalg.norm(oo), 1e-30))
    # how much of the tolerance the worst element uses (1.0 = at the bound)
    r_out = float((err_o / (OUT_TOL + OUT_TOL * np.abs(oo))).max())
    r_lse = float(np.nan_to_num(err_l / (LSE_TOL + LSE_TOL * np.abs(np.where(np.isinf(ol), 0.0, ol))),
                                nan=np.inf).max())
    print(f"[{label}] rows={len(sel)} max|dout|={err_o.max():.3e} rel_fro={rel_fro:.3e} "
          f"max|dlse|={err_l.max():.3e} max|out|={np.abs(oo).max():.3f} "
          f"worst err/tol out={r_out:.3f} lse={r_lse:.3f}", flush=True)
    record_margin(label=label, rows=int(len(sel)), max_dout=float(err_o.max()), rel_fro=rel_fro,
                  max_dlse=float(err_l.max()), max_abs_out=float(np.abs(oo).max()),
                  rms_out=float(np.sqrt(np.mean(oo ** 2))), worst_ratio_out=r_out, worst_ratio_lse=r_lse)
    assert (err_o <= OUT_TOL + OUT_TOL * np.abs(oo)).all(), f"{label}: out outside tolerance"
    assert (err_l <= LSE_TOL + LSE_TOL * np.abs(ol)).all(), f"{label}: lse outside tolerance"
    return g_out, g_lse


def record_margin(**rec):
    """Append one comparison's error figures to the JSON-lines file named by
    MTV_PARITY_LOG (if set); tests/conftest.py turns it into a table."""
    path = os.environ.get("MTV_PARITY_LOG")
    if path:
        import json
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def check_against(out, lse, o_out, o_lse, label):
    """Compare GPU (out, lse) tensors with oracle outputs, all rows."""
    g_out = out.view(torch.int16).cpu().numpy().view(np.uint16)
    g_lse = lse.cpu().numpy()

    class _Fixed:
        @staticmethod
        def run_workload(_wl, rows=None):
            return o_out, o_lse
    compare(None, _Fixed, label=label, gpu=(g_out, g_lse))


def sample_rows(wl, k, seed=0):
    total = wl.batch * wl.num_nodes * wl.num_heads
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, total - 1], rng.choice(total, size=min(k, total), replace=False)]))


# ----------------------------------------------------------- small, all rows

@pytest.mark.parametrize("q_gain", [1.0, 4.0])
def test_tiny_chain_all_rows(oracle_mod, q_gain):
    wl = I.config_workload(1, device="cuda", q_gain=q_gain)
    compare(wl, oracle_mod, label=f"chain8 ctx1024 gain{q_gain}")


@pytest.mark.parametrize("case", [
    dict(batch=1, num_nodes=9, num_heads=8, prefix_lens=[700], tree="random", max_depth=4),   # 72 rows
    dict(batch=1, num_nodes=16, num_heads=8, prefix_lens=[2000], tree="binary"),               # 128 rows
    dict(batch=3, num_nodes=5, num_heads=3, prefix_lens=[0, 31, 1000], tree="random", max_depth=3),
    dict(batch=2, num_nodes=64, num_heads=2, prefix_lens=[100, 4097], tree="random", max_depth=8),
    dict(batch=1, num_nodes=1, num_heads=1, prefix_lens=[0], tree="chain"),                    # one key
    dict(batch=2, num_nodes=8, num_heads=8, prefix_lens=[8191, 8193], tree="chain"),           # chunk edges
])
def test_small_shapes_all_rows(oracle_mod, case):
    wl = I.make_workload(num_slots=32768, config_id=100, device="cuda", **case)
    compare(wl, oracle_mod, label="B%d N%d H%d ctx%s %s" % (case["batch"], case["num_nodes"], case["num_heads"],
                                                            "/".join(map(str, case["prefix_lens"])), case["tree"]))


@pytest.mark.parametrize("n", [31, 32, 33, 64])
def test_random_bitmasks_word_boundaries(oracle_mod, n):
    m = I.random_bitmask(n, seed=500 + n, density=0.4)
    m[1, :] = 0  # node 1 sees only the prefix
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=4, prefix_lens=[77], num_slots=4096,
                         tree="chain", config_id=101, mask=m, device="cuda")
    compare(wl, oracle_mod, label=f"random bits n={n}")


def test_empty_visible_set(oracle_mod):
    m = np.array([[0], [3]], dtype=np.uint32)
    wl = I.make_workload(batch=1, num_nodes=2, num_heads=2, prefix_lens=[0], num_slots=64,
                         tree="chain", config_id=102, mask=m, device="cuda")
    g_out, g_lse = run_gpu(wl)
    assert np.all(g_out[0, 0] == 0) and np.all(np.isneginf(g_lse[0, 0]))
    compare(wl, oracle_mod, label="empty visible set")


# ---------------------------------------------------- bit-exact index / mask handling

def test_layout_invariance_bitwise():
    wl = I.make_workload(batch=3, num_nodes=8, num_heads=8, prefix_lens=[5000, 77, 12345],
                         num_slots=65536, tree="random", max_depth=5, config_id=104, device="cuda")
    ref = run_gpu(wl)
    for seed, layout in [(11, "scattered"), (12, "runs64")]:
        got = run_gpu(I.relayout(wl, seed, layout))
        assert np.array_equal(got[0], ref[0])
        assert np.array_equal(got[1].view(np.uint32), ref[1].view(np.uint32))


def test_repeat_runs_bitwise():
    wl = I.config_workload(1, device="cuda")
    a = run_gpu(wl)
    b = run_gpu(wl)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_masked_tree_rows_do_not_leak():
    n, h, ctx = 8, 8, 3000
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=h, prefix_lens=[ctx], num_slots=8192,
                         tree="chain", config_id=105, device="cuda")
    base = run_gpu(wl)
    slot = int(wl.page_table[0, ctx + n - 1].item())  # seen by node n-1 only
    poison = torch.tensor([1e4 if c % 2 == 0 else -1e4 for c in range(576)], device="cuda")
    wl.kv_pool[slot] = poison.to(torch.bfloat16)
    got = run_gpu(wl)
    assert np.array_equal(got[0][0, :n - 1], base[0][0, :n - 1])
    assert np.array_equal(got[1][0, :n - 1], base[1][0, :n - 1])
    assert not np.array_equal(got[0][0, n - 1], base[0][0, n - 1])


def test_positions_past_seq_len_are_not_read():
    wl = I.make_workload(batch=2, num_nodes=8, num_heads=8, prefix_lens=[100, 33], num_slots=4096,
                         tree="chain", config_id=106, max_kv=4000, device="cuda")
    base = run_gpu(wl)
    t = wl.page_table.clone()
    t[0, 108:] = 10 ** 9   # out of range: must never be gathered
    t[1, 41:] = -7
    wl.page_table = t
    got = run_gpu(wl)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])


@pytest.mark.parametrize("prefix", [3, 100, 3000, 39979])
def test_one_sequence_table_past_seq_len_is_not_read(oracle_mod, prefix):
    """One sequence whose plan covers max_kv keys: the table past its end
    names a NaN row (or an out-of-range slot, clamped to the pool's last
    row). The last tile's positions past the end must reuse a valid row; any
    use of the NaN row, even at weight zero, would make the outputs NaN. The
    lengths put the end in the first tile, mid-slice and near max_kv."""
    n, h, max_kv = 16, 8, 40000
    wl = I.make_workload(batch=1, num_nodes=n, num_heads=h, prefix_lens=[prefix], num_slots=65536,
                         tree="binary", config_id=113, device="cuda", max_kv=max_kv, q_gain=4.0)
    S = prefix + n
    base = run_gpu(wl)
    live = set(wl.page_table[0, :S].tolist())
    free = int(wl.page_table[0, S].item()) if S < max_kv else None
    assert free is not None and free not in live
    t = wl.page_table.clone()
    t[0, S + 40:] = 10 ** 9
    wl.page_table = t
    wl.kv_pool[free] = float("nan")
    if wl.num_slots - 1 not in live:
        wl.kv_pool[wl.num_slots - 1] = float("nan")
    got = run_gpu(wl)
    assert np.array_equal(got[0], base[0])
    assert np.array_equal(got[1].view(np.uint32), base[1].view(np.uint32))
    compare(wl, oracle_mod, rows=sample_rows(wl, 16, seed=prefix), label=f"table past S={S}",
            gpu=got)


# ------------------------------------------------------------ full-size configs

@pytest.mark.parametrize("q_gain", [1.0, 4.0])
def test_binary16_ctx65536(oracle_mod, q_gain):
    wl = I.config_workload(2, device="cuda", q_gain=q_gain)
    compare(wl, oracle_mod, label=f"binary16 ctx65536 gain{q_gain}")


@pytest.mark.parametrize("ctx", [1024, 11264, 32768, 65536, 131072, 189440])
def test_chain8_sweep_points(oracle_mod, ctx):
    """Every context of the 61-layer sweep: the first and the last layer (own
    pool and queries, the shared table), each at gains 1 and 4, all 64 rows."""
    for layer in (0, 60):
        for gain in (1.0, 4.0):
            wl = I.config_workload(3, device="cuda", ctx=ctx, layer=layer, q_gain=gain)
            compare(wl, oracle_mod, label=f"chain8 ctx{ctx} layer{layer} gain{gain}")
            del wl


def rows_per_group(wl, per_group, seed):
    """`per_group` distinct rows from every 64-row group, plus the first and last."""
    total = wl.batch * wl.num_nodes * wl.num_heads
    rng = np.random.default_rng(seed)
    pick = [0, total - 1]
    for g0 in range(0, total, 64):
        n = min(64, total - g0)
        pick.extend(g0 + rng.choice(n, size=min(per_group, n), replace=False))
    return np.unique(pick)


@pytest.mark.parametrize("q_gain,per_group", [(1.0, 4), (4.0, 1)])
def test_random64_h64_ctx131072(oracle_mod, q_gain, per_group):
    """64 nodes x 64 heads: 4096 rows in 64 row groups; rows drawn from every
    group (256 at gain 1, 64 at gain 4)."""
    wl = I.config_workload(4, device="cuda", q_gain=q_gain)
    rows = rows_per_group(wl, per_group, seed=4 + per_group)
    assert len(rows) >= 64 * per_group
    compare(wl, oracle_mod, rows=rows, label=f"random64 h64 ctx131072 gain{q_gain}")


@pytest.mark.parametrize("q_gain", [1.0, 4.0])
def test_batch8_both_layouts(oracle_mod, q_gain):
    """Batch 8, log-uniform contexts: all 512 rows against the oracle (at gain
    1 the 34k-59k-key sequences have outputs near the absolute tolerance, so
    gain 4 is the sharp check), and the runs-of-64 relayout bit for bit."""
    a = I.config_workload(5, device="cuda", layout="scattered", q_gain=q_gain)
    ga = run_gpu(a)
    compare(a, oracle_mod, label=f"batch8 scattered gain{q_gain}", gpu=ga)
    b = I.relayout(a, I.seed_for(5, 0, I.F_TABLE) + 1, "runs64")
    gb = run_gpu(b)
    assert np.array_equal(ga[0], gb[0]) and np.array_equal(ga[1], gb[1])


def test_long_slices_restage_index_window(oracle_mod):
    """Several row groups leave few, long slices: with 7 row groups (64 nodes x
    7 heads, one row group per workgroup) over 160k keys a slice spans more
    than one 128-tile window of staged page indices, so the kernel restages
    indices inside its tile loop. (From 8 row groups on, slices that long run
    two row groups per workgroup; their restage is covered by the 64 x 64-head
    tests.)"""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=7, prefix_lens=[160000], num_slots=262144,
                         tree="random", max_depth=8, config_id=107, device="cuda", q_gain=4.0)
    plan = M.plan_query(M.make_shape(1, 64, 7, wl.max_kv, wl.num_slots),
                        torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["row_groups"] == 7 and plan["chunk"] > 128 * 32, plan
    compare(wl, oracle_mod, rows=sample_rows(wl, 64, seed=7), label="long slices")


# ------------------------------------------------- length-balanced slicing of a batch

def test_uneven_batch_balanced_slices(oracle_mod):
    """One long sequence among short ones: the long one is cut into many
    slices, each short one into one; every row against the oracle."""
    wl = I.make_workload(batch=5, num_nodes=4, num_heads=4, prefix_lens=[30000, 3, 100, 0, 2500],
                         num_slots=65536, tree="random", max_depth=3, config_id=108, device="cuda",
                         q_gain=4.0)
    compare(wl, oracle_mod, label="uneven batch")


@pytest.mark.parametrize("batch", [64, 65, 100, 256, 300, 600])
def test_many_sequences(oracle_mod, batch):
    """The edges of the slicing paths: one sequence per lane up to 64, then
    the split kernel's block-wide slicing, with one sequence per thread up to
    256 and a loop over the batch beyond."""
    rng = np.random.default_rng(batch)
    pre = [int(x) for x in rng.integers(0, 90, size=batch)]
    pre[batch // 2] = 4000  # one long sequence takes several slices
    wl = I.make_workload(batch=batch, num_nodes=2, num_heads=2, prefix_lens=pre, num_slots=65536,
                         tree="chain", config_id=109, device="cuda")
    compare(wl, oracle_mod, label=f"{batch} sequences")


def test_batch_sequence_with_many_slices(oracle_mod):
    """A batch whose long sequence has more slices than one round of the batch
    combine's waves holds (8 waves x 16 slices in flight): its merge runs two
    rounds per wave."""
    pre = [150000, 500]
    wl = I.make_workload(batch=2, num_nodes=8, num_heads=8, prefix_lens=pre, num_slots=262144,
                         tree="chain", config_id=111, device="cuda", q_gain=4.0)
    # the device's slicing: c tiles per slice, c = ceil(T / (G - (B - 1))) for G slots
    G = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = [(p + 8 + 31) // 32 for p in pre]
    c = -(-sum(tiles) // (G - 1))
    assert -(-tiles[0] // c) > 8 * 16
    compare(wl, oracle_mod, rows=sample_rows(wl, 32, seed=11), label="batch, 247-slice sequence")


def test_one_sequence_shorter_than_max_kv_ignores_stale_workspace(oracle_mod):
    """One sequence with far fewer keys than max_kv: the plan has slices for
    max_kv, the combine loads all of them, and the ones this call did not
    write (here a workspace of NaN bytes) must get no weight."""
    wl = I.make_workload(batch=1, num_nodes=16, num_heads=8, prefix_lens=[3000], num_slots=65536,
                         tree="binary", config_id=112, device="cuda", max_kv=40000, q_gain=4.0)
    shape = M.make_shape(1, 16, 8, wl.max_kv, wl.num_slots)
    plan = M.plan_query(shape, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["splits"] * plan["chunk"] >= 40000 and plan["chunk"] < 3016 // 4
    ws = torch.full((M.workspace_size(shape),), 0xFF, dtype=torch.uint8, device="cuda")
    out, lse = M.verify_workload(wl, workspace=ws)
    torch.cuda.synchronize()
    compare(wl, oracle_mod, label="short sequence, NaN workspace",
            gpu=(out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()))


def test_batch_slicing_is_independent_of_layout_and_padding():
    """The slicing depends only on seq_lens: the same batch with a larger
    max_kv (more table columns, junk past every sequence) gives the same bits."""
    wl = I.make_workload(batch=4, num_nodes=8, num_heads=8, prefix_lens=[9000, 40, 700, 20000],
                         num_slots=65536, tree="binary", config_id=110, device="cuda")
    a = run_gpu(wl)
    wide = torch.full((4, wl.max_kv + 5000), 10 ** 9, dtype=torch.int32, device="cuda")
    wide[:, :wl.max_kv] = wl.page_table
    wl.page_table = wide
    b = run_gpu(wl)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ------------------------------------------------------------------ graph capture

def test_graph_capture_replays_match_eager():
    wl = I.make_workload(batch=2, num_nodes=16, num_heads=8, prefix_lens=[3000, 9000],
                         num_slots=32768, tree="binary", config_id=107, device="cuda")
    eager_out, eager_lse = M.verify_workload(wl)
    torch.cuda.synchronize()
    eager = (eager_out.clone(), eager_lse.clone())
    shape = M.make_shape(wl.batch, wl.num_nodes, wl.num_heads, wl.max_kv, wl.num_slots)
    ws = torch.empty(M.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(eager_out)
    lse = torch.empty_like(eager_lse)
    other = I.config_workload(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.verify_workload(wl, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.verify_workload(wl, out=out, lse=lse, workspace=ws)
    for _ in range(4):
        out.fill_(0)
        lse.fill_(0)
        g.replay()
        M.verify_workload(other)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16))
        assert torch.equal(lse, eager[1])


def test_captured_multi_layer_step_with_mask_build(oracle_mod):
    """A verify step captured as one graph: the mask build from the parent
    array, then 6 layers (own pool and queries, one shared page table and
    workspace). The device-built mask equals the tree-mask oracle's; the first
    and the last layer of the first replay match the attention oracle (peaked
    queries, every row); every replay, with eager work in between, equals
    eager bit for bit."""
    from oracle import tree_mask as T
    base = I.make_workload(batch=1, num_nodes=16, num_heads=8, prefix_lens=[7000],
                           num_slots=16384, tree="random", max_depth=5, config_id=109, device="cuda")
    parents_np = np.ascontiguousarray(base.parents, dtype=np.int32)
    parents = torch.from_numpy(parents_np).cuda()
    mask = torch.zeros_like(base.tree_mask)
    layers = [I.make_workload(batch=1, num_nodes=16, num_heads=8, prefix_lens=[7000],
                              num_slots=16384, tree="random", max_depth=5, config_id=109,
                              layer=l, device="cuda", q_gain=4.0) for l in range(6)]
    ws = None
    calls = []
    for wl in layers:
        c = M.PreparedCall(wl.q, wl.kv_pool, base.page_table, base.seq_lens, mask, wl.scale,
                           workspace=ws)
        ws = c.workspace
        calls.append(c)

    def step():
        M.tree_mask_build(parents, out=mask)
        for c in calls:
            c.run()

    step()
    torch.cuda.synchronize()
    oracle_mask = T.tree_mask(parents_np[None] if parents_np.ndim == 1 else parents_np)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), oracle_mask)
    eager = [(c.out.clone(), c.lse.clone()) for c in calls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = I.config_workload(1, device="cuda")
    for rep in range(3):
        mask.zero_()
        for c in calls:
            c.out.zero_()
            c.lse.zero_()
        g.replay()
        M.verify_workload(other)  # eager work between replays
        torch.cuda.synchronize()
        if rep == 0:
            for l in (0, len(layers) - 1):
                wl = layers[l]
                o_out, o_lse = oracle_mod.run(wl.np_q(), wl.np_kv(), base.np_page_table(),
                                              base.np_seq_lens(), oracle_mask, wl.scale)
                check_against(calls[l].out, calls[l].lse, o_out, o_lse, f"captured step layer {l}")
        for c, (o, l) in zip(calls, eager):
            assert torch.equal(c.out.view(torch.int16), o.view(torch.int16))
            assert torch.equal(c.lse.view(torch.int32), l.view(torch.int32))
