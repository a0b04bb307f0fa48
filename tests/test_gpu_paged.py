"""GPU parity of the hybrid-paging entry point (mla_tree_verify_paged).

The CPU side expands (prefix_pages, tree_slots) into a per-token table with
oracle/hybrid_table.py and runs the attention oracle on it; tolerances are the
attention's (out 2e-2 abs + rel, lse 1e-3 abs + rel). The GPU side is also
checked bit for bit against mla_tree_verify on the expanded table, since both
read the same rows in the same order.
"""
import time

import numpy as np
import pytest
import torch

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import inputs as I
from oracle import hybrid_table as H

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    M.load()


def bits_to_f64(t):
    b = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def run_paged(wl, pages, tree, page_size):
    out, lse = M.mla_tree_verify_paged(wl.q, wl.kv_pool, pages, tree, wl.seq_lens, wl.tree_mask,
                                       wl.scale, page_size, wl.max_kv)
    torch.cuda.synchronize()
    return out, lse


def run_per_token(wl, table):
    out, lse = M.mla_tree_verify(wl.q, wl.kv_pool, table, wl.seq_lens, wl.tree_mask, wl.scale)
    torch.cuda.synchronize()
    return out, lse


def oracle_expand(wl, pages, tree, page_size):
    return H.expand(pages.cpu().numpy(), tree.cpu().numpy(), wl.seq_lens_host(), wl.num_nodes,
                    page_size, wl.max_kv)


def check_vs_oracle(oracle_mod, wl, table, out, lse, rows=None, label=""):
    o_out, o_lse = oracle_mod.run(wl.np_q(), wl.np_kv(), table, wl.np_seq_lens(), wl.np_mask(),
                                  wl.scale, rows=rows)
    go = bits_to_f64(out).reshape(-1, 512)
    oo = (o_out.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 512)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    ol = o_lse.astype(np.float64).reshape(-1)
    sel = np.arange(gl.size) if rows is None else np.asarray(rows)
    eo = np.abs(go[sel] - oo[sel])
    el = np.abs(gl[sel] - ol[sel])
    print(f"[{label}] rows={len(sel)} max|dout|={eo.max():.3e} max|dlse|={el.max():.3e}", flush=True)
    assert np.isfinite(go[sel]).all()
    assert (eo <= OUT_TOL + OUT_TOL * np.abs(oo[sel])).all(), label
    assert (el <= LSE_TOL + LSE_TOL * np.abs(ol[sel])).all(), label


def check_bitwise(wl, pages, tree, page_size, table):
    po, pl = run_paged(wl, pages, tree, page_size)
    to, tl = run_per_token(wl, torch.from_numpy(table).to(wl.q.device))
    assert torch.equal(po.view(torch.int16), to.view(torch.int16))
    assert torch.equal(pl.view(torch.int32), tl.view(torch.int32))
    return po, pl


@pytest.mark.parametrize("page_size", [1, 16, 64, 256])
def test_small_all_rows(oracle_mod, page_size):
    # ragged prefixes: 1000 and 37 are not multiples of any page size here but 1
    wl = I.make_workload(batch=3, num_nodes=8, num_heads=4, prefix_lens=[1000, 37, 4100],
                         num_slots=16384, tree="binary", config_id=21, device="cuda")
    hl = I.hybrid_layout(wl, page_size, seed=3 + page_size)
    w = hl.workload
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, page_size)
    out, lse = check_bitwise(w, hl.prefix_pages, hl.tree_slots, page_size, table)
    check_vs_oracle(oracle_mod, w, table, out, lse, label=f"paged{page_size} small")


def test_no_prefix(oracle_mod):
    # t0 = 0: every visible key is a tree node; the page list is never read
    wl = I.make_workload(batch=2, num_nodes=16, num_heads=8, prefix_lens=[0, 5],
                         num_slots=1024, tree="random", config_id=22, device="cuda")
    hl = I.hybrid_layout(wl, 64, seed=1)
    w = hl.workload
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, 64)
    out, lse = check_bitwise(w, hl.prefix_pages, hl.tree_slots, 64, table)
    check_vs_oracle(oracle_mod, w, table, out, lse, label="paged no prefix")


def test_short_page_list_reads_last_entry(oracle_mod):
    # a prefix longer than max_pages * page_size reads the row's last page again
    wl = I.make_workload(batch=1, num_nodes=8, num_heads=8, prefix_lens=[300],
                         num_slots=4096, tree="chain", config_id=23, device="cuda",
                         poison_unreferenced=False)  # hand-picked pages read any row
    dev = wl.q.device
    pages = torch.tensor([[7, 2, 11]], dtype=torch.int32, device=dev)  # covers 192 of 300
    tree = torch.tensor([[900 + 3 * i for i in range(8)]], dtype=torch.int32, device=dev)
    table = oracle_expand(wl, pages, tree, 64)
    assert (table[0, 192:300] // 64 == 11).all()
    out, lse = check_bitwise(wl, pages, tree, 64, table)
    check_vs_oracle(oracle_mod, wl, table, out, lse, label="paged short list")


def test_invalid_pages_clamp_like_the_table():
    # negative or out-of-pool pages give slots that both entry points clamp to
    # the pool the same way; the output is finite and bit-identical
    wl = I.make_workload(batch=2, num_nodes=8, num_heads=8, prefix_lens=[500, 700],
                         num_slots=8192, tree="chain", config_id=24, device="cuda",
                         poison_unreferenced=False)
    dev = wl.q.device
    g = np.random.default_rng(5)
    pages = g.integers(0, 128, size=(2, 11)).astype(np.int32)
    pages[0, 3] = -1
    pages[1, 5] = 128 + 40  # beyond the pool's 128 pages
    tree = g.integers(0, 8192, size=(2, 8)).astype(np.int32)
    tree[1, 2] = -5
    pages_t = torch.from_numpy(pages).to(dev)
    tree_t = torch.from_numpy(tree).to(dev)
    table = oracle_expand(wl, pages_t, tree_t, 64)
    out, lse = check_bitwise(wl, pages_t, tree_t, 64, table)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("page_size", [64, 1024])
def test_batch8_loguniform_sampled(oracle_mod, page_size):
    wl = I.config_workload(5, device="cuda")
    hl = I.hybrid_layout(wl, page_size, seed=page_size)
    w = hl.workload
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, page_size)
    out, lse = check_bitwise(w, hl.prefix_pages, hl.tree_slots, page_size, table)
    total = w.batch * w.num_nodes * w.num_heads
    rows = np.unique(np.concatenate([[0, total - 1],
                                     np.random.default_rng(page_size).choice(total, 48, replace=False)]))
    check_vs_oracle(oracle_mod, w, table, out, lse, rows=rows, label=f"batch8 paged{page_size}")
    # the relaid logical inputs give the same attention as the original layout
    ro, rl = run_per_token(wl, wl.page_table)
    assert torch.equal(ro.view(torch.int16), out.view(torch.int16))


def test_graph_capture_paged():
    """Captured paged call: every replay, with eager work between replays,
    equals the eager call."""
    wl = I.config_workload(2, device="cuda")
    hl = I.hybrid_layout(wl, 64, seed=9)
    w = hl.workload
    ref_o, ref_l = run_paged(w, hl.prefix_pages, hl.tree_slots, 64)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    ws = torch.empty(M.workspace_size(M.make_shape(w.batch, w.num_nodes, w.num_heads, w.max_kv,
                                                   w.num_slots)), dtype=torch.uint8, device="cuda")

    def call():
        M.mla_tree_verify_paged(w.q, w.kv_pool, hl.prefix_pages, hl.tree_slots, w.seq_lens,
                                w.tree_mask, w.scale, 64, w.max_kv, out=out, lse=lse, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other = I.config_workload(1, device="cuda")
    for _ in range(3):
        out.zero_()
        lse.zero_()
        g.replay()
        M.verify_workload(other)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))


@pytest.mark.parametrize("page_size", [48, 100])
def test_page_size_not_a_power_of_two(oracle_mod, page_size):
    # page numbers by division rather than a shift; ragged last pages
    wl = I.make_workload(batch=2, num_nodes=9, num_heads=8, prefix_lens=[5000, 777],
                         num_slots=16384, tree="random", max_depth=4, config_id=25, device="cuda")
    hl = I.hybrid_layout(wl, page_size, seed=page_size)
    w = hl.workload
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, page_size)
    out, lse = check_bitwise(w, hl.prefix_pages, hl.tree_slots, page_size, table)
    check_vs_oracle(oracle_mod, w, table, out, lse, label=f"paged{page_size}")


def test_long_slices_restage_paged_window(oracle_mod):
    """7 row groups (64 nodes x 7 heads) over 160k keys leave slices of more
    than one 4096-position window, so the hybrid layout's index staging runs
    again inside the tile loop; bit for bit equal to the per-token call on the
    expanded table, which runs the same one-row-group plan here."""
    wl = I.make_workload(batch=1, num_nodes=64, num_heads=7, prefix_lens=[160000], num_slots=262144,
                         tree="random", max_depth=8, config_id=107, device="cuda", q_gain=4.0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = M.plan_query(M.make_shape(1, 64, 7, wl.max_kv, wl.num_slots), cus)
    assert plan["row_groups"] == 7 and plan["chunk"] > 4096, plan
    hl = I.hybrid_layout(wl, 64, seed=5)
    w = hl.workload
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, 64)
    out, lse = check_bitwise(w, hl.prefix_pages, hl.tree_slots, 64, table)
    rows = np.unique(np.r_[0, 447, np.random.default_rng(3).choice(448, 40, replace=False)])
    check_vs_oracle(oracle_mod, w, table, out, lse, rows=rows, label="paged long slices")


def test_prepared_paged_call_matches_the_call():
    """PreparedPagedCall.run (pointers marshalled once) gives the bits of
    mla_tree_verify_paged, on every repeat."""
    wl = I.config_workload(5, device="cuda")
    hl = I.hybrid_layout(wl, 64, seed=64)
    w = hl.workload
    ref_o, ref_l = run_paged(w, hl.prefix_pages, hl.tree_slots, 64)
    call = M.PreparedPagedCall(w.q, w.kv_pool, hl.prefix_pages, hl.tree_slots, w.seq_lens, w.tree_mask,
                               w.scale, 64, w.max_kv)
    for _ in range(3):
        call.out.zero_()
        call.lse.zero_()
        call.run()
        torch.cuda.synchronize()
        assert torch.equal(call.out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(call.lse.view(torch.int32), ref_l.view(torch.int32))


def test_many_rows_long_slices_keep_one_row_group(oracle_mod):
    """64 nodes x 64 heads at 131072 keys under hybrid paging: the per-token
    plan runs two row groups per workgroup here, the hybrid call keeps one
    (its own slicing), and the one workspace size serves both."""
    wl = I.config_workload(4, device="cuda", q_gain=4.0)
    hl = I.hybrid_layout(wl, 64, seed=4)
    w = hl.workload
    per_token_splits = M.plan_query(M.make_shape(1, 64, 64, w.max_kv, w.num_slots),
                                    torch.cuda.get_device_properties(0).multi_processor_count)["splits"]
    out, lse = run_paged(w, hl.prefix_pages, hl.tree_slots, 64)
    table = oracle_expand(w, hl.prefix_pages, hl.tree_slots, 64)
    rng = np.random.default_rng(41)
    rows = np.unique(np.r_[0, 4095, [g * 64 + rng.integers(64) for g in range(64)]])
    check_vs_oracle(oracle_mod, w, table, out, lse, rows=rows, label=f"paged64 h64 (per-token plan {per_token_splits} slices)")


def test_per_token_first_calls_after_idle_match_paged():
    """Per-token calls (the two-kinds-of-wave split kernel) made right after
    the GPU sat idle, each the first call on freshly built inputs with peaked
    queries (Q x 4, so running maxima are raised in late tiles), against the
    hybrid-paging call on the same rows, bit for bit. A rescale flag written
    to LDS just before a barrier, with no wait for the write, made about one
    such call in nine wrong."""
    for k in range(8):
        if k % 2 == 0:
            wl = I.config_workload(2, device="cuda", q_gain=4.0, layer=k // 2)
        else:
            wl = I.config_workload(3, device="cuda", ctx=32768 if k % 4 == 1 else 65536, layer=k, q_gain=4.0)
        hl = I.hybrid_layout(wl, 64, seed=100 + k)
        w = hl.workload
        table = torch.from_numpy(oracle_expand(w, hl.prefix_pages, hl.tree_slots, 64)).to(w.q.device)
        torch.cuda.synchronize()
        time.sleep(1.0)
        to, tl = run_per_token(w, table)
        po, pl = run_paged(w, hl.prefix_pages, hl.tree_slots, 64)
        assert torch.equal(to.view(torch.int16), po.view(torch.int16)), f"call {k}: out differs"
        assert torch.equal(tl.view(torch.int32), pl.view(torch.int32)), f"call {k}: lse differs"
        del wl, hl, w, table
