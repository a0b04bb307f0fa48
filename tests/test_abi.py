"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad host-side arguments before touching a device."""
import ctypes
import os
import re

import pytest

import mla_tree_verify_02_amd as M
from mla_tree_verify_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_tree_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = M.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert M.status_string(code) and M.status_string(code) != "unknown status"
    assert M.status_string(-99) == "unknown status"


@pytest.mark.parametrize("shape,ok", [
    ((1, 8, 8, 1032, 4096), True),
    ((8, 64, 64, 131136, 1 << 21), True),
    ((0, 8, 8, 1032, 4096), False),       # no sequences
    ((1, 0, 8, 1032, 4096), False),       # no tree
    ((1, 65, 8, 1032, 4096), False),      # more than two mask words
    ((1, 8, 0, 1032, 4096), False),
    ((1, 64, 1025, 1032, 4096), False),   # more than 65536 query rows
    ((1, 8, 8, 7, 4096), False),          # max_kv below the tree size
    ((1, 8, 8, 1032, 0), False),
    ((1, 8, 8, 1032, 1 << 31), False),    # slot indices are int32
])
def test_workspace_size_validates_shape(shape, ok):
    ws = M.workspace_size(M.make_shape(*shape))
    assert (ws > 0) == ok


@pytest.mark.parametrize("b,n,h,max_kv,cus", [
    (1, 8, 8, 1032, 256), (1, 16, 8, 65552, 256), (1, 64, 64, 131136, 256),
    (8, 8, 8, 131080, 256), (1, 8, 8, 189448, 256), (1, 1, 1, 1, 256), (3, 9, 8, 777, 32),
])
def test_plan_covers_every_key(b, n, h, max_kv, cus):
    p = M.plan_query(M.make_shape(b, n, h, max_kv, 1 << 20), cus)
    tiles = (max_kv + 31) // 32
    assert p["chunk"] % 32 == 0 and 32 <= p["chunk"] <= 32 * tiles
    assert p["splits"] * p["chunk"] >= max_kv
    assert (p["splits"] - 1) * p["chunk"] < max_kv
    assert p["row_groups"] == (n * h + 63) // 64
    # about one workgroup per compute unit whenever there is that much work
    # (rounding the slices to whole tiles can lose up to half of it)
    pairs = b * p["row_groups"]
    assert pairs * p["splits"] >= min(cus, pairs * tiles) // 2


@pytest.mark.parametrize("n,h,max_kv,splits", [
    (64, 64, 131136, 8),    # 64 row groups, 513-tile slices: two row groups per workgroup
    (64, 17, 131136, 29),   # 17 row groups (9 workgroup groups), 142-tile slices: two
    (64, 16, 65600, 32),    # 16 row groups, 65-tile slices: two
    (64, 16, 49216, 32),    # 49-tile slices: two
    (64, 16, 40992, 16),    # two would give 41-tile slices: one (81-tile slices)
    (64, 16, 32800, 16),    # two would give 33-tile slices: one
    (64, 64, 8256, 4),      # two would give 33-tile slices: one
    (64, 8, 131136, 64),    # 8 row groups, 65-tile slices: two
    (64, 8, 98368, 32),     # 8 row groups: two would give 49-tile slices, one
    (64, 7, 131136, 37),    # 7 row groups: one
    (16, 8, 65552, 121),    # 2 row groups: one
])
def test_two_row_group_plan_rule(n, h, max_kv, splits):
    """Two 64-row groups share a split workgroup from 16 row groups and 48
    tiles per slice, or from 8 row groups and 64 tiles: on 256 CUs the slot
    count then doubles."""
    p = M.plan_query(M.make_shape(1, n, h, max_kv, 1 << 20), 256)
    assert p["splits"] == splits, p


def test_noalloc_scratch_covers_one_sequence_of_up_to_32768_rows():
    for h in (64, 128, 512):
        for kv in (1024, 131136, 1 << 22):
            assert M.workspace_size(M.make_shape(1, 64, h, kv, 1 << 20)) <= _lib.NOALLOC_SCRATCH_BYTES


def _call(shape, ptrs=None, ws_bytes=1 << 30, scale=0.07):
    lib = M.load()
    good = 1 << 20  # a 256-byte-aligned stand-in address; never dereferenced on the host
    p = dict(q=good, kv=good, pt=good, sl=good, tm=good, out=good, lse=good, ws=good)
    if ptrs:
        p.update(ptrs)
    V = ctypes.c_void_p
    return lib.mla_tree_verify(ctypes.byref(shape), V(p["q"]), V(p["kv"]), V(p["pt"]),
                               V(p["sl"]), V(p["tm"]), ctypes.c_float(scale), V(p["out"]),
                               V(p["lse"]), V(p["ws"]), ctypes.c_size_t(ws_bytes), None)


def test_null_pointers_rejected():
    s = M.make_shape(1, 8, 8, 1032, 4096)
    for k in ("q", "kv", "pt", "sl", "tm", "out", "lse", "ws"):
        assert _call(s, {k: None}) == -1, k
    assert M.load().mla_tree_verify(None, None, None, None, None, None, ctypes.c_float(1.0),
                                    None, None, None, 0, None) == -1


def test_bad_shape_and_scale_rejected():
    assert _call(M.make_shape(1, 65, 8, 1032, 4096)) == -2
    assert _call(M.make_shape(1, 8, 8, 1032, 4096), scale=float("nan")) == -2
    assert _call(M.make_shape(1, 8, 8, 1032, 4096), scale=float("inf")) == -2


def test_misalignment_rejected():
    s = M.make_shape(1, 8, 8, 1032, 4096)
    base = 1 << 20
    for k, off in (("q", 8), ("kv", 2), ("out", 4), ("pt", 2), ("sl", 1), ("tm", 2),
                   ("lse", 2), ("ws", 64)):
        assert _call(s, {k: base + off}) == -3, k


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 8, 8, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        M.mla_tree_verify(q, torch.zeros(16, 576, dtype=torch.bfloat16),
                          torch.zeros(1, 16, dtype=torch.int32), torch.tensor([16], dtype=torch.int32),
                          torch.zeros(1, 8, 1, dtype=torch.int32), 0.1)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(FileNotFoundError):
        _lib.load(str(tmp_path / "nope.so"))


def test_tree_mask_build_rejects_bad_arguments():
    lib = M.load()
    V = ctypes.c_void_p
    good = 1 << 20
    assert lib.mla_tree_mask_build(1, 8, None, V(good), None) == -1
    assert lib.mla_tree_mask_build(1, 8, V(good), None, None) == -1
    for b, n in [(0, 8), (1, 0), (1, 65), (70000, 8)]:
        assert lib.mla_tree_mask_build(b, n, V(good), V(good), None) == -2
    assert lib.mla_tree_mask_build(1, 8, V(good + 2), V(good), None) == -3
    assert lib.mla_tree_mask_build(1, 8, V(good), V(good + 1), None) == -3


def test_kv_moves_reject_bad_arguments():
    lib = M.load()
    V = ctypes.c_void_p
    g = V(1 << 20)
    # commit: NULLs, shapes, alignment
    assert lib.mla_kv_commit(1, 8, 100, 1000, None, g, g, g, g, g, None) == -1
    assert lib.mla_kv_commit(1, 8, 100, 1000, g, g, g, g, None, g, None) == -1
    for b, n, mkv, p in [(0, 8, 100, 1000), (1, 0, 100, 1000), (1, 65, 100, 1000), (1, 8, 7, 1000),
                         (1, 8, 100, 0), (1, 8, 100, 1 << 31)]:
        assert lib.mla_kv_commit(b, n, mkv, p, g, g, g, g, g, g, None) == -2
    assert lib.mla_kv_commit(1, 8, 100, 1000, V((1 << 20) + 8), g, g, g, g, g, None) == -3
    assert lib.mla_kv_commit(1, 8, 100, 1000, g, V((1 << 20) + 2), g, g, g, g, None) == -3
    # defrag
    assert lib.mla_kv_defrag(1, 100, 1000, g, None, g, g, None) == -1
    for b, mkv, p in [(0, 100, 1000), (1, 0, 1000), (1, 100, 0)]:
        assert lib.mla_kv_defrag(b, mkv, p, g, g, g, g, None) == -2
    assert lib.mla_kv_defrag(1, 100, 1000, V((1 << 20) + 4), g, g, g, None) == -3


def test_paged_entry_rejects_bad_arguments():
    lib = M.load()
    V = ctypes.c_void_p
    g = 1 << 20
    s = M.make_shape(1, 8, 8, 1032, 4096)

    def call(ps=64, mp=17, pages=g, tree=g, q=g, scale=0.07):
        return lib.mla_tree_verify_paged(ctypes.byref(s), ps, mp, V(q), V(g), V(pages), V(tree),
                                         V(g), V(g), ctypes.c_float(scale), V(g), V(g), V(g),
                                         ctypes.c_size_t(1 << 30), None)

    assert call(pages=None) == -1
    assert call(tree=None) == -1
    assert call(q=None) == -1
    for ps, mp in [(0, 17), (-64, 17), (64, 0), (64, -1), (1 << 30, 17)]:
        assert call(ps=ps, mp=mp) == -2, (ps, mp)
    assert call(scale=float("nan")) == -2
    assert call(pages=g + 2) == -3
    assert call(tree=g + 1) == -3


def test_input_check_rejects_bad_arguments():
    lib = M.load()
    V = ctypes.c_void_p
    g = 1 << 20

    def call(shape=(1, 8, 8, 1032, 4096), pt=g, sl=g, mk=g, counts=g):
        s = M.make_shape(*shape)
        return lib.mtv_check_inputs(ctypes.byref(s), V(pt), V(sl), V(mk), V(counts), None)

    assert lib.mtv_check_inputs(None, V(g), V(g), V(g), V(g), None) == -1
    assert call(pt=None) == -1
    assert call(counts=None) == -1
    for shape in [(0, 8, 8, 1032, 4096), (1, 0, 8, 1032, 4096), (1, 65, 8, 1032, 4096),
                  (1, 8, 8, 7, 4096), (1, 8, 8, 1032, 0), (1, 8, 8, 1032, 1 << 31)]:
        assert call(shape=shape) == -2, shape
    assert call(sl=g + 2) == -3
    assert call(counts=g + 4) == -3   # the counters are 64-bit
