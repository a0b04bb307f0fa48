"""ctypes binding of libmla_tree_verify.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels. This module
checks torch tensors' dtypes, shapes, devices and contiguity, hands their device
pointers and the current HIP stream to the C ABI, and turns a status code into
an exception. There is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import LIB_PATH

MTV_OK = 0
STATUS_NAMES = {0: "MTV_OK", -1: "MTV_ERR_NULL", -2: "MTV_ERR_SHAPE", -3: "MTV_ERR_ALIGN",
                -4: "MTV_ERR_WORKSPACE", -5: "MTV_ERR_HIP", -6: "MTV_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # MTV_NOALLOC_SCRATCH_BYTES
EXPORTED = ("mla_tree_verify", "mla_tree_verify_workspace_size", "mtv_status_string",
            "mtv_plan_query", "mla_tree_verify_splitkv", "mla_tree_verify_combine",
            "mla_tree_mask_build", "mla_kv_commit", "mla_kv_defrag", "mla_tree_verify_paged",
            "mtv_check_inputs", "mla_tree_verify_noalloc")


class MtvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_nodes", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("max_kv", ctypes.c_int32),
                ("num_slots", ctypes.c_int64)]


class MtvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: Optional[str] = None):
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m mla_tree_verify_02_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    VP = ctypes.c_void_p
    SP = ctypes.POINTER(MtvShape)
    lib.mla_tree_verify.restype = ctypes.c_int
    lib.mla_tree_verify.argtypes = [SP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP, VP,
                                    ctypes.c_size_t, VP]
    lib.mla_tree_verify_noalloc.restype = ctypes.c_int
    lib.mla_tree_verify_noalloc.argtypes = [SP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP, VP]
    lib.mla_tree_verify_splitkv.restype = ctypes.c_int
    lib.mla_tree_verify_splitkv.argtypes = [SP, VP, VP, VP, VP, VP, ctypes.c_float, VP,
                                            ctypes.c_size_t, VP]
    lib.mla_tree_verify_combine.restype = ctypes.c_int
    lib.mla_tree_verify_combine.argtypes = [SP, VP, VP, VP, VP, ctypes.c_size_t, VP]
    lib.mla_tree_verify_workspace_size.restype = ctypes.c_size_t
    lib.mla_tree_verify_workspace_size.argtypes = [SP]
    lib.mtv_status_string.restype = ctypes.c_char_p
    lib.mtv_status_string.argtypes = [ctypes.c_int]
    lib.mtv_plan_query.restype = ctypes.c_int
    IP = ctypes.POINTER(ctypes.c_int)
    lib.mtv_plan_query.argtypes = [SP, ctypes.c_int, IP, IP, IP]
    lib.mla_tree_mask_build.restype = ctypes.c_int
    lib.mla_tree_mask_build.argtypes = [ctypes.c_int32, ctypes.c_int32, VP, VP, VP]
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    lib.mla_tree_verify_paged.restype = ctypes.c_int
    lib.mla_tree_verify_paged.argtypes = [SP, I32, I32, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP,
                                          VP, VP, ctypes.c_size_t, VP]
    lib.mla_kv_commit.restype = ctypes.c_int
    lib.mla_kv_commit.argtypes = [I32, I32, I32, I64, VP, VP, VP, VP, VP, VP, VP]
    lib.mla_kv_defrag.restype = ctypes.c_int
    lib.mla_kv_defrag.argtypes = [I32, I32, I64, VP, VP, VP, VP, VP]
    lib.mtv_check_inputs.restype = ctypes.c_int
    lib.mtv_check_inputs.argtypes = [SP, VP, VP, VP, VP, VP]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mtv_status_string(int(status)).decode()


def make_shape(batch: int, num_nodes: int, num_heads: int, max_kv: int, num_slots: int) -> MtvShape:
    return MtvShape(int(batch), int(num_nodes), int(num_heads), int(max_kv), int(num_slots))


def workspace_size(shape: MtvShape) -> int:
    return int(load().mla_tree_verify_workspace_size(ctypes.byref(shape)))


def plan_query(shape: MtvShape, num_cus: int):
    """The slicing mtv_plan_query reports for a batch whose sequences all hold
    max_kv keys: slices per sequence, keys per slice, 64-row groups."""
    s, c, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = load().mtv_plan_query(ctypes.byref(shape), int(num_cus), ctypes.byref(s),
                               ctypes.byref(c), ctypes.byref(g))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return {"splits": s.value, "chunk": c.value, "row_groups": g.value}


def _check(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def mla_tree_verify(q: torch.Tensor, kv_pool: torch.Tensor, page_table: torch.Tensor,
                    seq_lens: torch.Tensor, tree_mask: torch.Tensor, scale: float,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """Tree-verify attention through the C ABI (same argument order and names).

    q bf16 [B,N,H,576]; kv_pool bf16 [P,576]; page_table int32 [B,max_kv];
    seq_lens int32 [B]; tree_mask int32/uint32 bit patterns [B,N,ceil(N/32)].
    Returns (out bf16 [B,N,H,512], lse float32 [B,N,H]). Runs asynchronously on
    `stream` (default: torch's current stream on q's device).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, 576]")
    B, N, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    if D != 576:
        raise ValueError("q rows must be 576 wide")
    if kv_pool.dim() != 2:
        raise ValueError("kv_pool must be [num_slots, 576]")
    P = kv_pool.shape[0]
    if page_table.dim() != 2:
        raise ValueError("page_table must be [B, max_kv]")
    max_kv = page_table.shape[1]
    W = (N + 31) // 32
    _check(q, "q", torch.bfloat16, (B, N, H, 576), dev)
    _check(kv_pool, "kv_pool", torch.bfloat16, (P, 576), dev)
    _check(page_table, "page_table", torch.int32, (B, max_kv), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if tree_mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("tree_mask must hold 32-bit words")
    _check(tree_mask, "tree_mask", tree_mask.dtype, (B, N, W), dev)
    if out is None:
        out = torch.empty((B, N, H, 512), dtype=torch.bfloat16, device=dev)
    else:
        _check(out, "out", torch.bfloat16, (B, N, H, 512), dev)
    if lse is None:
        lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (B, N, H), dev)
    shape = make_shape(B, N, H, max_kv, P)
    lib = load()
    with torch.cuda.device(dev):
        need = int(lib.mla_tree_verify_workspace_size(ctypes.byref(shape)))
        if need == 0:
            raise MtvError(-2, status_string(-2))
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        handle = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
        rc = lib.mla_tree_verify(ctypes.byref(shape), _ptr(q), _ptr(kv_pool), _ptr(page_table),
                                 _ptr(seq_lens), _ptr(tree_mask), ctypes.c_float(scale), _ptr(out),
                                 _ptr(lse), _ptr(workspace),
                                 ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                 handle)
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return out, lse


def mla_tree_verify_noalloc(q: torch.Tensor, kv_pool: torch.Tensor, page_table: torch.Tensor,
                            seq_lens: torch.Tensor, tree_mask: torch.Tensor, scale: float,
                            out: torch.Tensor, lse: torch.Tensor, stream=None):
    """mla_tree_verify without a workspace argument: the library's fixed
    per-GPU scratch holds the partials (see mla_tree_verify_noalloc). The
    caller passes preallocated out bf16 [B,N,H,512] and lse float32 [B,N,H];
    nothing is allocated here either. Returns (out, lse)."""
    if q.dim() != 4 or page_table.dim() != 2 or kv_pool.dim() != 2:
        raise ValueError("q must be [B, N, H, 576], page_table [B, max_kv], kv_pool [P, 576]")
    B, N, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    P = kv_pool.shape[0]
    max_kv = page_table.shape[1]
    _check(q, "q", torch.bfloat16, (B, N, H, 576), dev)
    _check(kv_pool, "kv_pool", torch.bfloat16, (P, 576), dev)
    _check(page_table, "page_table", torch.int32, (B, max_kv), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if tree_mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("tree_mask must hold 32-bit words")
    _check(tree_mask, "tree_mask", tree_mask.dtype, (B, N, (N + 31) // 32), dev)
    _check(out, "out", torch.bfloat16, (B, N, H, 512), dev)
    _check(lse, "lse", torch.float32, (B, N, H), dev)
    shape = make_shape(B, N, H, max_kv, P)
    lib = load()
    with torch.cuda.device(dev):
        rc = lib.mla_tree_verify_noalloc(ctypes.byref(shape), _ptr(q), _ptr(kv_pool), _ptr(page_table),
                                         _ptr(seq_lens), _ptr(tree_mask), ctypes.c_float(scale),
                                         _ptr(out), _ptr(lse), _stream_handle(dev, stream))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return out, lse


def tree_mask_build(parents: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """Ancestor-or-self visibility bitmask from a parent array, built by the
    library's kernel.

    parents int32 [B, N] on a GPU (parent of node i in [-1, i), -1 for roots;
    other values are read as -1). Returns int32 bit patterns [B, N, ceil(N/32)]
    in the layout mla_tree_verify takes as tree_mask.
    """
    if parents.dim() != 2:
        raise ValueError("parents must be [B, N]")
    B, N = parents.shape
    dev = parents.device
    if dev.type != "cuda":
        raise ValueError("parents must be on a GPU")
    _check(parents, "parents", torch.int32, (B, N), dev)
    W = (N + 31) // 32
    if out is None:
        out = torch.empty((B, N, W), dtype=torch.int32, device=dev)
    else:
        if out.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
            raise TypeError("out must hold 32-bit words")
        _check(out, "out", out.dtype, (B, N, W), dev)
    lib = load()
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        handle = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
        rc = lib.mla_tree_mask_build(ctypes.c_int32(B), ctypes.c_int32(N), _ptr(parents), _ptr(out),
                                     handle)
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return out


def mla_tree_verify_paged(q: torch.Tensor, kv_pool: torch.Tensor, prefix_pages: torch.Tensor,
                          tree_slots: torch.Tensor, seq_lens: torch.Tensor, tree_mask: torch.Tensor,
                          scale: float, page_size: int, max_kv: int,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Tree-verify attention with hybrid paging (see mla_tree_verify_paged):
    prefix_pages int32 [B, max_pages] (pages of page_size slots), tree_slots
    int32 [B, N]; max_kv bounds every sequence length. Returns (out, lse)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, 576]")
    B, N, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    if kv_pool.dim() != 2 or prefix_pages.dim() != 2:
        raise ValueError("kv_pool must be [num_slots, 576] and prefix_pages [B, max_pages]")
    P = kv_pool.shape[0]
    max_pages = prefix_pages.shape[1]
    W = (N + 31) // 32
    _check(q, "q", torch.bfloat16, (B, N, H, 576), dev)
    _check(kv_pool, "kv_pool", torch.bfloat16, (P, 576), dev)
    _check(prefix_pages, "prefix_pages", torch.int32, (B, max_pages), dev)
    _check(tree_slots, "tree_slots", torch.int32, (B, N), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if tree_mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("tree_mask must hold 32-bit words")
    _check(tree_mask, "tree_mask", tree_mask.dtype, (B, N, W), dev)
    if out is None:
        out = torch.empty((B, N, H, 512), dtype=torch.bfloat16, device=dev)
    else:
        _check(out, "out", torch.bfloat16, (B, N, H, 512), dev)
    if lse is None:
        lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (B, N, H), dev)
    shape = make_shape(B, N, H, max_kv, P)
    lib = load()
    with torch.cuda.device(dev):
        need = int(lib.mla_tree_verify_workspace_size(ctypes.byref(shape)))
        if need == 0:
            raise MtvError(-2, status_string(-2))
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        rc = lib.mla_tree_verify_paged(ctypes.byref(shape), int(page_size), int(max_pages), _ptr(q),
                                       _ptr(kv_pool), _ptr(prefix_pages), _ptr(tree_slots),
                                       _ptr(seq_lens), _ptr(tree_mask), ctypes.c_float(scale),
                                       _ptr(out), _ptr(lse), _ptr(workspace),
                                       ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                       _stream_handle(dev, stream))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return out, lse


def _stream_handle(dev, stream):
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def kv_commit(kv_pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
              num_nodes: int, accept_len: torch.Tensor, accept_path: torch.Tensor,
              region_base: torch.Tensor, stream=None) -> None:
    """Move each sequence's accepted tree nodes into its contiguous run of
    slots and update the page table in place (see mla_kv_commit)."""
    dev = kv_pool.device
    if dev.type != "cuda":
        raise ValueError("kv_pool must be on a GPU")
    if kv_pool.dim() != 2 or page_table.dim() != 2:
        raise ValueError("kv_pool must be [num_slots, 576] and page_table [B, max_kv]")
    P = kv_pool.shape[0]
    B, max_kv = page_table.shape
    N = int(num_nodes)
    _check(kv_pool, "kv_pool", torch.bfloat16, (P, 576), dev)
    _check(page_table, "page_table", torch.int32, (B, max_kv), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _check(accept_len, "accept_len", torch.int32, (B,), dev)
    _check(accept_path, "accept_path", torch.int32, (B, N), dev)
    _check(region_base, "region_base", torch.int32, (B,), dev)
    lib = load()
    with torch.cuda.device(dev):
        rc = lib.mla_kv_commit(B, N, max_kv, P, _ptr(kv_pool), _ptr(page_table), _ptr(seq_lens),
                               _ptr(accept_len), _ptr(accept_path), _ptr(region_base),
                               _stream_handle(dev, stream))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))


def kv_defrag(kv_pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
              region_base: torch.Tensor, stream=None) -> None:
    """Move every sequence's rows to region_base[b] + position and rewrite the
    page table in place (see mla_kv_defrag)."""
    dev = kv_pool.device
    if dev.type != "cuda":
        raise ValueError("kv_pool must be on a GPU")
    if kv_pool.dim() != 2 or page_table.dim() != 2:
        raise ValueError("kv_pool must be [num_slots, 576] and page_table [B, max_kv]")
    P = kv_pool.shape[0]
    B, max_kv = page_table.shape
    _check(kv_pool, "kv_pool", torch.bfloat16, (P, 576), dev)
    _check(page_table, "page_table", torch.int32, (B, max_kv), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _check(region_base, "region_base", torch.int32, (B,), dev)
    lib = load()
    with torch.cuda.device(dev):
        rc = lib.mla_kv_defrag(B, max_kv, P, _ptr(kv_pool), _ptr(page_table), _ptr(seq_lens),
                               _ptr(region_base), _stream_handle(dev, stream))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))


def check_inputs(page_table: torch.Tensor, seq_lens: torch.Tensor, tree_mask: torch.Tensor,
                 num_slots: int, counts: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Count out-of-range device inputs of mla_tree_verify on the GPU (see
    mtv_check_inputs): returns int64 [3] on the device, (bad sequence
    lengths, bad table entries below each clamped length, mask rows with bits
    past the last node). Asynchronous: read it after the stream gets there."""
    dev = page_table.device
    if dev.type != "cuda":
        raise ValueError("page_table must be on a GPU")
    if page_table.dim() != 2 or tree_mask.dim() != 3:
        raise ValueError("page_table must be [B, max_kv] and tree_mask [B, N, W]")
    B, max_kv = page_table.shape
    N = tree_mask.shape[1]
    _check(page_table, "page_table", torch.int32, (B, max_kv), dev)
    _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if tree_mask.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError("tree_mask must hold 32-bit words")
    _check(tree_mask, "tree_mask", tree_mask.dtype, (B, N, (N + 31) // 32), dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int64, device=dev)
    else:
        _check(counts, "counts", torch.int64, (3,), dev)
    shape = make_shape(B, N, 1, max_kv, num_slots)
    lib = load()
    with torch.cuda.device(dev):
        rc = lib.mtv_check_inputs(ctypes.byref(shape), _ptr(page_table), _ptr(seq_lens),
                                  _ptr(tree_mask), _ptr(counts), _stream_handle(dev, stream))
    if rc != MTV_OK:
        raise MtvError(rc, status_string(rc))
    return counts


def verify_workload(wl, **kw):
    """Run on an ``inputs.Workload`` whose tensors are on a GPU."""
    return mla_tree_verify(wl.q, wl.kv_pool, wl.page_table, wl.seq_lens, wl.tree_mask,
                           wl.scale, **kw)


class PreparedCall:
    """Validated, preallocated arguments of one call, for repeated launches.

    Holds the workspace and the outputs so that ``run()``, ``splitkv()`` and
    ``combine()`` only marshal pointers into the C ABI (as a benchmark or a
    captured graph needs). Tensors must stay alive and unchanged in shape.
    """

    def __init__(self, q, kv_pool, page_table, seq_lens, tree_mask, scale, workspace=None):
        B, N, H, _ = q.shape
        dev = q.device
        self.out = torch.empty((B, N, H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
        self.shape = make_shape(B, N, H, page_table.shape[1], kv_pool.shape[0])
        need = workspace_size(self.shape)
        if need == 0:
            raise MtvError(-2, status_string(-2))
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.inputs = (q, kv_pool, page_table, seq_lens, tree_mask)
        self.scale = float(scale)
        self.device = dev
        # one validating call through the full binding
        mla_tree_verify(q, kv_pool, page_table, seq_lens, tree_mask, scale, out=self.out,
                        lse=self.lse, workspace=self.workspace)
        self._lib = load()
        self._p = [ctypes.c_void_p(t.data_ptr()) for t in self.inputs]
        self._out = ctypes.c_void_p(self.out.data_ptr())
        self._lse = ctypes.c_void_p(self.lse.data_ptr())
        self._ws = ctypes.c_void_p(self.workspace.data_ptr())
        self._wsb = ctypes.c_size_t(self.workspace.numel() * self.workspace.element_size())

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def run(self):
        q, kv, pt, sl, tm = self._p
        rc = self._lib.mla_tree_verify(ctypes.byref(self.shape), q, kv, pt, sl, tm,
                                       ctypes.c_float(self.scale), self._out, self._lse, self._ws,
                                       self._wsb, self._stream())
        if rc != MTV_OK:
            raise MtvError(rc, status_string(rc))

    def splitkv(self):
        q, kv, pt, sl, tm = self._p
        rc = self._lib.mla_tree_verify_splitkv(ctypes.byref(self.shape), q, kv, pt, sl, tm,
                                               ctypes.c_float(self.scale), self._ws, self._wsb,
                                               self._stream())
        if rc != MTV_OK:
            raise MtvError(rc, status_string(rc))

    def combine(self):
        rc = self._lib.mla_tree_verify_combine(ctypes.byref(self.shape), self._p[3], self._out,
                                               self._lse, self._ws, self._wsb, self._stream())
        if rc != MTV_OK:
            raise MtvError(rc, status_string(rc))


class PreparedPagedCall:
    """PreparedCall for the hybrid layout (mla_tree_verify_paged): one
    validating call through the full binding, then ``run()`` only marshals the
    held pointers."""

    def __init__(self, q, kv_pool, prefix_pages, tree_slots, seq_lens, tree_mask, scale, page_size,
                 max_kv, workspace=None):
        B, N, H, _ = q.shape
        dev = q.device
        self.out = torch.empty((B, N, H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
        self.shape = make_shape(B, N, H, max_kv, kv_pool.shape[0])
        need = workspace_size(self.shape)
        if need == 0:
            raise MtvError(-2, status_string(-2))
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.inputs = (q, kv_pool, prefix_pages, tree_slots, seq_lens, tree_mask)
        self.scale = float(scale)
        self.page_size = int(page_size)
        self.max_pages = int(prefix_pages.shape[1])
        self.device = dev
        mla_tree_verify_paged(q, kv_pool, prefix_pages, tree_slots, seq_lens, tree_mask, scale,
                              page_size, max_kv, out=self.out, lse=self.lse, workspace=self.workspace)
        self._lib = load()
        self._p = [ctypes.c_void_p(t.data_ptr()) for t in self.inputs]
        self._out = ctypes.c_void_p(self.out.data_ptr())
        self._lse = ctypes.c_void_p(self.lse.data_ptr())
        self._ws = ctypes.c_void_p(self.workspace.data_ptr())
        self._wsb = ctypes.c_size_t(self.workspace.numel() * self.workspace.element_size())

    def run(self):
        q, kv, pp, ts, sl, tm = self._p
        rc = self._lib.mla_tree_verify_paged(ctypes.byref(self.shape), self.page_size, self.max_pages, q,
                                             kv, pp, ts, sl, tm, ctypes.c_float(self.scale), self._out,
                                             self._lse, self._ws, self._wsb,
                                             ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream))
        if rc != MTV_OK:
            raise MtvError(rc, status_string(rc))


def prepare_workload(wl, workspace=None) -> PreparedCall:
    return PreparedCall(wl.q, wl.kv_pool, wl.page_table, wl.seq_lens, wl.tree_mask, wl.scale,
                        workspace=workspace)
