"""Hybrid paging as a per-token page table (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; it shares no code with the HIP library.

The pages propose larger pages for the prefix while the draft tree stays
fine-grained ("The 130x Slowdown: Diagnosing Latency-Bound Decode in
Speculative Decoding on Blackwell GPUs", The Broader Implications: What This
Diagnosis Means). The reading taken: prefix position p (p < t0 = S - N) of sequence
b lives at prefix_pages[b][p // page_size] * page_size + p % page_size (a page
number beyond the row reads the row's last entry), tree node n at
tree_slots[b][n]. Expanding that into the per-token table of the verify
attention is the whole of the hybrid path's definition; the attention itself
is the (separately pinned) oracle in oracle.py.
"""
from __future__ import annotations

import numpy as np


def expand(prefix_pages: np.ndarray, tree_slots: np.ndarray, seq_lens, num_nodes: int,
           page_size: int, max_kv: int) -> np.ndarray:
    """int32 [B, max_kv] per-token table; entries at positions >= S_b are 0."""
    prefix_pages = np.asarray(prefix_pages, dtype=np.int64)
    tree_slots = np.asarray(tree_slots, dtype=np.int64)
    B, max_pages = prefix_pages.shape
    N = int(num_nodes)
    out = np.zeros((B, max_kv), dtype=np.int64)
    for b in range(B):
        S = min(max(int(seq_lens[b]), N), max_kv)
        t0 = S - N
        for p in range(t0):
            page = prefix_pages[b, min(p // page_size, max_pages - 1)]
            out[b, p] = page * page_size + p % page_size
        for n in range(N):
            out[b, t0 + n] = tree_slots[b, n]
    return out.astype(np.int32)
