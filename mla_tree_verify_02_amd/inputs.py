"""Seeded synthetic workloads for the absorbed-MLA tree-verify attention step.

This module draws random numbers and lays out buffers; it holds none of the
attention arithmetic. Both the CPU oracle and the HIP path are fed from what it
builds, so a test can hand the very same bytes to each side.

What a workload is made of (the pages' statement of the problem):
  * a latent KV pool with one token per page ("page_size=1"), each row a bf16
    512-d latent followed by a 64-d RoPE key (1152 bytes) -- "The 130x Slowdown",
    section The Technical Depth, and "The Moment of Doubt", quoted message (13 GB
    of compressed latents over 61 layers at 185k);
  * a per-token page table that the kernel gathers through -- "The 130x
    Slowdown", The Reasoning, step 4;
  * a small draft tree of query nodes (about nine) whose tree block must be
    masked while the long prefix needs no mask -- "The Moment of Certainty",
    sections Message 12190 and The Path Forward;
  * a per-node tree visibility bitmask -- "The GPU That Wasn't There", section
    The Native Engine Thesis.

Layout conventions (shared with the C ABI):
  q          bf16  [B, N, H, 576]   absorbed query: q_latent[512] | q_rope[64]
  kv_pool    bf16  [P, 576]         latent[512] | rope_k[64]
  page_table int32 [B, max_kv]      positions [0, S_b - N) are the prefix,
                                    positions [S_b - N, S_b) are tree nodes 0..N-1
  seq_lens   int32 [B]              S_b = prefix length + N
  tree_mask  uint32 [B, N, W]       W = ceil(N / 32); bit (j & 31) of word (j >> 5)
                                    of node i set <=> node i may attend node j
Unreferenced pool slots hold bf16 NaN so that any stray read poisons the result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE
ROW_BYTES = D_QK * 2
BF16_NAN_BITS = 0x7FC0
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

# Seed fields: one stream per kind of input so that changing one shape does not
# perturb the others.
F_KV, F_Q, F_TABLE, F_TREE, F_LENS, F_POISON = 0, 1, 2, 3, 4, 5


def seed_for(config_id: int, layer: int, fld: int) -> int:
    """Seed of one input stream: 1_000_000 * config + 1000 * layer + field."""
    return 1_000_000 * int(config_id) + 1000 * int(layer) + int(fld)


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


# --------------------------------------------------------------------------- trees

def chain_parents(n: int) -> np.ndarray:
    """A chain of n nodes: node i hangs under node i - 1 (node 0 is the root)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def heap_binary_parents(n: int) -> np.ndarray:
    """Binary tree in heap order: parent[i] = (i - 1) // 2."""
    p = (np.arange(n, dtype=np.int64) - 1) // 2
    p[0] = -1
    return p.astype(np.int32)


def random_parents(n: int, max_depth: int, seed: int) -> np.ndarray:
    """Random tree with parent[i] < i and depth <= max_depth (root depth 0).

    parent[i] is drawn uniformly among the earlier nodes whose depth is at most
    max_depth - 1, so that no node goes deeper than max_depth.
    """
    g = _gen(seed, "cpu")
    parents = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        cand = np.nonzero(depth[:i] <= max_depth - 1)[0]
        k = int(torch.randint(len(cand), (1,), generator=g).item())
        parents[i] = cand[k]
        depth[i] = depth[cand[k]] + 1
    return parents


def tree_depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int32)
    for i in range(len(parents)):
        d[i] = 0 if parents[i] < 0 else d[parents[i]] + 1
    return d


def mask_words(n: int) -> int:
    return (n + 31) // 32


def ancestor_bitmask(parents: np.ndarray) -> np.ndarray:
    """uint32 [N, W]: node i's bits are itself and all of its ancestors."""
    n = len(parents)
    w = mask_words(n)
    m = np.zeros((n, w), dtype=np.uint32)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j >> 5] |= np.uint32(1 << (j & 31))
            j = int(parents[j])
    return m


def random_bitmask(n: int, seed: int, density: float = 0.5) -> np.ndarray:
    """uint32 [N, W] with independent random bits for j < n (bits >= n zero)."""
    g = _gen(seed, "cpu")
    bits = (torch.rand((n, n), generator=g) < density).numpy()
    m = np.zeros((n, mask_words(n)), dtype=np.uint32)
    for i in range(n):
        for j in range(n):
            if bits[i, j]:
                m[i, j >> 5] |= np.uint32(1 << (j & 31))
    return m


# ---------------------------------------------------------------------- workloads

@dataclass
class Workload:
    """One call's worth of inputs, on one device (CPU or GPU)."""

    q: torch.Tensor            # bf16 [B, N, H, 576]
    kv_pool: torch.Tensor      # bf16 [P, 576]
    page_table: torch.Tensor   # int32 [B, max_kv]
    seq_lens: torch.Tensor     # int32 [B]
    tree_mask: torch.Tensor    # int32 [B, N, W] holding uint32 bit patterns
    parents: np.ndarray        # int32 [B, N] tree topology used to build the mask
    scale: float
    prefix_lens: List[int] = field(default_factory=list)
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_nodes(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def max_kv(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_slots(self) -> int:
        return int(self.kv_pool.shape[0])

    def seq_lens_host(self) -> List[int]:
        return [p + self.num_nodes for p in self.prefix_lens]

    def to(self, device: str) -> "Workload":
        return Workload(self.q.to(device), self.kv_pool.to(device),
                        self.page_table.to(device), self.seq_lens.to(device),
                        self.tree_mask.to(device), self.parents.copy(), self.scale,
                        list(self.prefix_lens), self.name)

    # numpy views in the C ABI's byte formats (for the oracle)
    def np_q(self) -> np.ndarray:
        return self.q.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def np_kv(self) -> np.ndarray:
        return self.kv_pool.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def np_page_table(self) -> np.ndarray:
        return self.page_table.detach().cpu().contiguous().numpy().astype(np.int32, copy=False)

    def np_seq_lens(self) -> np.ndarray:
        return self.seq_lens.detach().cpu().contiguous().numpy().astype(np.int32, copy=False)

    def np_mask(self) -> np.ndarray:
        return self.tree_mask.detach().cpu().contiguous().numpy().view(np.uint32)


def _randn_bf16(shape, gen: torch.Generator, device: str, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to bf16, generated in row chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen,
                                  device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def scattered_table(seq_lens: Sequence[int], num_slots: int, seed: int):
    """Fully fragmented page_size=1 layout: a seeded permutation of the pool,
    sequence b taking the next S_b slots of it (disjoint across sequences).
    Returns (per-sequence slot arrays, unreferenced slots)."""
    g = _gen(seed, "cpu")
    perm = torch.randperm(num_slots, generator=g).numpy().astype(np.int32)
    total = int(sum(seq_lens))
    if total > num_slots:
        raise ValueError("pool too small for the sequences")
    table = []
    off = 0
    for s in seq_lens:
        table.append(perm[off:off + s])
        off += s
    return table, perm[off:]


def contiguous_run_table(seq_lens: Sequence[int], num_slots: int, seed: int,
                         run: int = 64):
    """page_size=64 style layout expressed as a per-token table: tokens fill
    runs of `run` slots inside run-aligned pages taken from a seeded page
    permutation. Returns (per-sequence slot arrays, unreferenced slots)."""
    g = _gen(seed, "cpu")
    npages = num_slots // run
    pperm = torch.randperm(npages, generator=g).numpy().astype(np.int64)
    table = []
    pg = 0
    for s in seq_lens:
        need = (s + run - 1) // run
        if pg + need > npages:
            raise ValueError("pool too small for the sequences")
        pages = pperm[pg:pg + need]
        t = np.arange(s, dtype=np.int64)
        table.append((pages[t // run] * run + t % run).astype(np.int32))
        pg += need
    used = np.zeros(num_slots, dtype=bool)
    for t in table:
        used[t] = True
    return table, np.nonzero(~used)[0].astype(np.int32)


def make_workload(*, batch: int = 1, num_nodes: int = 8, num_heads: int = 8,
                  prefix_lens: Sequence[int] = (1024,), num_slots: int = 4096,
                  tree: str = "chain", max_depth: int = 8, layout: str = "scattered",
                  config_id: int = 1, layer: int = 0, scale: float = DEFAULT_SCALE,
                  q_gain: float = 1.0, max_kv: Optional[int] = None,
                  device: str = "cpu", poison_unreferenced: bool = True,
                  mask: Optional[np.ndarray] = None, kv_seed: Optional[int] = None,
                  table_seed: Optional[int] = None, name: str = "") -> Workload:
    """Build one seeded workload.

    tree: "chain" | "binary" | "random" (parent[i] < i, depth <= max_depth)
    layout: "scattered" (random permutation) | "runs64" (contiguous runs of 64)
    q_gain: multiplies Q after rounding (a power of two keeps it exact in bf16);
            4 gives the "peaked" variant whose outputs are O(0.1-1) at long context.
    mask: optional explicit uint32 [N, W] (or [B, N, W]) bitmask overriding the tree's.
    """
    prefix_lens = [int(p) for p in prefix_lens]
    if len(prefix_lens) != batch:
        raise ValueError("prefix_lens must have one entry per sequence")
    n, h = int(num_nodes), int(num_heads)
    seq = [p + n for p in prefix_lens]
    mkv = max(seq) if max_kv is None else int(max_kv)
    if mkv < max(seq):
        raise ValueError("max_kv smaller than the longest sequence")

    # tree topology and bitmask
    parents = np.zeros((batch, n), dtype=np.int32)
    for b in range(batch):
        if tree == "chain":
            parents[b] = chain_parents(n)
        elif tree == "binary":
            parents[b] = heap_binary_parents(n)
        elif tree == "random":
            parents[b] = random_parents(n, max_depth, seed_for(config_id, layer, F_TREE) + 17 * b)
        else:
            raise ValueError(f"unknown tree {tree!r}")
    w = mask_words(n)
    if mask is None:
        m = np.stack([ancestor_bitmask(parents[b]) for b in range(batch)])
    else:
        m = np.asarray(mask, dtype=np.uint32)
        if m.ndim == 2:
            m = np.broadcast_to(m, (batch, n, w)).copy()
    if m.shape != (batch, n, w):
        raise ValueError("mask shape mismatch")

    # page table
    tseed = seed_for(config_id, 0, F_TABLE) if table_seed is None else table_seed
    if layout == "scattered":
        rows, spare = scattered_table(seq, num_slots, tseed)
    elif layout == "runs64":
        rows, spare = contiguous_run_table(seq, num_slots, tseed)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    tail_fill = int(spare[0]) if len(spare) else 0
    table = np.full((batch, mkv), tail_fill, dtype=np.int32)
    for b in range(batch):
        table[b, :seq[b]] = rows[b]

    # values
    kseed = seed_for(config_id, layer, F_KV) if kv_seed is None else kv_seed
    gdev = "cuda" if device.startswith("cuda") else "cpu"
    kv = _randn_bf16((num_slots, D_QK), _gen(kseed, gdev), device)
    if poison_unreferenced and len(spare):
        sp = torch.from_numpy(spare.astype(np.int64)).to(device)
        kv.view(torch.int16)[sp] = torch.tensor(BF16_NAN_BITS, dtype=torch.int16, device=device)
    q = _randn_bf16((batch * n * h, D_QK), _gen(seed_for(config_id, layer, F_Q), gdev), device)
    q = q.view(batch, n, h, D_QK)
    if q_gain != 1.0:
        q = (q.float() * q_gain).to(torch.bfloat16)

    return Workload(
        q=q, kv_pool=kv,
        page_table=torch.from_numpy(table).to(device),
        seq_lens=torch.tensor(seq, dtype=torch.int32, device=device),
        tree_mask=torch.from_numpy(m.view(np.int32).copy()).to(device),
        parents=parents, scale=float(scale), prefix_lens=prefix_lens, name=name)


# ------------------------------------------------------------- the named configs

def log_uniform_prefixes(batch: int, lo: int, hi: int, seed: int) -> List[int]:
    """Seeded context lengths, log-uniform in [lo, hi]."""
    g = _gen(seed, "cpu")
    u = torch.rand(batch, generator=g, dtype=torch.float64).numpy()
    return [int(math.floor(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]


CONTEXTS_SWEEP = (1024, 11264, 32768, 65536, 131072, 189440)


def config_workload(cid: int, *, device: str = "cpu", layer: int = 0, ctx: Optional[int] = None,
                    layout: str = "scattered", q_gain: float = 1.0) -> Workload:
    """Workloads shaped like the five configurations.

    1: tiny chain, B1 N8 H8, context 1024, pool 4096
    2: B1 N16 (binary, depth 4) H8, context 65536, pool 262144
    3: B1 N8 chain H8, one layer of the 61-layer sweep at context `ctx`, pool 262144
    4: B1 N64 random tree (depth <= 8) H64, context 131072, pool 262144
    5: B8 N8 chain H8, log-uniform contexts in [1024, 131072], pool 2^21,
       layout "scattered" or "runs64"
    """
    if cid == 1:
        return make_workload(batch=1, num_nodes=8, num_heads=8, prefix_lens=[1024],
                             num_slots=4096, tree="chain", config_id=1, layer=layer,
                             device=device, q_gain=q_gain, name="tiny-chain-ctx1024")
    if cid == 2:
        return make_workload(batch=1, num_nodes=16, num_heads=8, prefix_lens=[65536],
                             num_slots=262144, tree="binary", config_id=2, layer=layer,
                             device=device, q_gain=q_gain, name="binary16-ctx65536")
    if cid == 3:
        c = 65536 if ctx is None else int(ctx)
        # one page table for every layer (seeded by config only), values per layer
        return make_workload(batch=1, num_nodes=8, num_heads=8, prefix_lens=[c],
                             num_slots=262144, tree="chain", config_id=3, layer=layer,
                             device=device, q_gain=q_gain,
                             table_seed=seed_for(3, 0, F_TABLE) + c,
                             name=f"chain8-ctx{c}-layer{layer}")
    if cid == 4:
        return make_workload(batch=1, num_nodes=64, num_heads=64, prefix_lens=[131072],
                             num_slots=262144, tree="random", max_depth=8, config_id=4,
                             layer=layer, device=device, q_gain=q_gain,
                             name="random64-h64-ctx131072")
    if cid == 5:
        pre = log_uniform_prefixes(8, 1024, 131072, seed_for(5, 0, F_LENS))
        return make_workload(batch=8, num_nodes=8, num_heads=8, prefix_lens=pre,
                             num_slots=1 << 21, tree="chain", config_id=5, layer=layer,
                             layout=layout, device=device, q_gain=q_gain,
                             table_seed=seed_for(5, 0, F_TABLE) + (1 if layout == "runs64" else 0),
                             name=f"batch8-loguniform-{layout}")
    raise ValueError(f"unknown config {cid}")


def relayout(wl: Workload, table_seed: int, layout: str) -> Workload:
    """The same logical inputs under another page table: every referenced KV row
    moves to the slot the new table (`layout`, seeded by `table_seed`) gives its
    position; Q, mask, lengths and scale are unchanged; unreferenced slots hold
    NaN. Runs on the workload's device."""
    other = make_workload(batch=wl.batch, num_nodes=wl.num_nodes, num_heads=wl.num_heads,
                          prefix_lens=wl.prefix_lens, num_slots=wl.num_slots, tree="chain",
                          layout=layout, table_seed=table_seed, config_id=0,
                          mask=wl.np_mask(), device=str(wl.q.device),
                          name=f"{wl.name}-{layout}")
    other.q = wl.q.clone()
    other.scale = wl.scale
    old = wl.kv_pool.view(torch.int16)
    new = torch.full_like(old, BF16_NAN_BITS)
    t_old, t_new = wl.page_table.long(), other.page_table.long()
    for b, s in enumerate(wl.seq_lens_host()):
        new[t_new[b, :s]] = old[t_old[b, :s]]
    other.kv_pool = new.view(torch.bfloat16)
    return other


@dataclass
class HybridLayout:
    """A workload's rows under hybrid paging: prefix positions in pages of
    page_size slots, tree nodes at scattered slots. `workload` holds the
    relaid pool and the equivalent per-token table."""
    workload: Workload
    prefix_pages: torch.Tensor  # int32 [B, max_pages]
    tree_slots: torch.Tensor    # int32 [B, N]
    page_size: int


def hybrid_layout(wl: Workload, page_size: int, seed: int) -> HybridLayout:
    """The same logical inputs with the prefix of each sequence in whole pages
    of `page_size` slots (page numbers from a seeded permutation of the pool's
    pages) and its N tree rows at seeded scattered slots outside those pages.
    Unreferenced slots hold NaN; unused page entries are 0."""
    P = wl.num_slots
    g = _gen(seed, "cpu")
    npages = P // page_size
    pperm = torch.randperm(npages, generator=g).numpy().astype(np.int64)
    N = wl.num_nodes
    seqs = wl.seq_lens_host()
    max_pages = max(1, max((s - N + page_size - 1) // page_size for s in seqs))
    pages = np.zeros((wl.batch, max_pages), dtype=np.int64)
    used = np.zeros(P, dtype=bool)
    pg = 0
    for b, s in enumerate(seqs):
        need = (s - N + page_size - 1) // page_size
        if pg + need > npages:
            raise ValueError("pool too small for the prefixes")
        pages[b, :need] = pperm[pg:pg + need]
        for q in pperm[pg:pg + need]:
            used[q * page_size:(q + 1) * page_size] = True
        pg += need
    free = np.nonzero(~used)[0]
    free = free[torch.randperm(len(free), generator=g).numpy()]
    if len(free) < wl.batch * N:
        raise ValueError("pool too small for the tree rows")
    tree = free[:wl.batch * N].reshape(wl.batch, N)
    table = np.zeros((wl.batch, wl.max_kv), dtype=np.int64)
    for b, s in enumerate(seqs):
        t0 = s - N
        p = np.arange(t0)
        table[b, :t0] = pages[b, p // page_size] * page_size + p % page_size
        table[b, t0:s] = tree[b]
        table[b, s:] = tree[b, 0]  # never read (positions >= S)
    dev = wl.q.device
    old = wl.kv_pool.view(torch.int16)
    new = torch.full_like(old, BF16_NAN_BITS)
    t_old = wl.page_table.long()
    t_new = torch.from_numpy(table).to(dev)
    for b, s in enumerate(seqs):
        new[t_new[b, :s]] = old[t_old[b, :s]]
    out = Workload(q=wl.q.clone(), kv_pool=new.view(torch.bfloat16),
                   page_table=t_new.to(torch.int32), seq_lens=wl.seq_lens.clone(),
                   tree_mask=wl.tree_mask.clone(), parents=wl.parents, scale=wl.scale,
                   prefix_lens=list(wl.prefix_lens), name=f"{wl.name}-paged{page_size}")
    return HybridLayout(out, torch.from_numpy(pages.astype(np.int32)).to(dev),
                        torch.from_numpy(tree.astype(np.int32)).to(dev), page_size)


def algorithmic_bytes(seq_lens: Sequence[int], num_nodes: int, num_heads: int) -> int:
    """Bytes a call must move at minimum: every referenced 1152-byte KV row once
    and its 4-byte page index, Q in, out and lse out, and the mask."""
    b = len(seq_lens)
    r = num_nodes * num_heads
    w = mask_words(num_nodes)
    return (sum(int(s) for s in seq_lens) * (ROW_BYTES + 4)
            + b * r * (D_QK * 2 + D_LATENT * 2 + 4) + b * num_nodes * w * 4)


def algorithmic_flops(seq_lens: Sequence[int], num_nodes: int, num_heads: int) -> int:
    """Dense-contraction flops: 2 * rows * (576 + 512) per key, per sequence."""
    r = num_nodes * num_heads
    return sum(2 * r * (D_QK + D_LATENT) * int(s) for s in seq_lens)
