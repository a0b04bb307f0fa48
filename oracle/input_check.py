"""CPU oracle of the verify attention's input check (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; it shares no code with the HIP library.

What it computes: for the three index inputs the attention reads from device
memory -- the per-token page table ("The 130x Slowdown", The Reasoning, step
4), the sequence lengths S_b = prefix + N (the tree block sits at the end of
each sequence, "The Moment of Certainty", The User Provides the Final Piece)
and the per-node tree bitmask ("The Moment of Certainty", The Path Forward) --
how many values lie outside the ranges the attention assumes:
  [0] sequences b with seq_lens[b] outside [N, max_kv];
  [1] entries page_table[b][p] outside [0, num_slots), for p < S_b where S_b
      is seq_lens[b] clamped to [N, max_kv] (the positions the attention reads);
  [2] mask rows (b, i) with a bit set for a node j >= N.
The pages state the ranges but no check; counting per category is the reading
taken here. Method: the definition, one Python loop per category.
"""
from __future__ import annotations

import numpy as np


def check_inputs(page_table, seq_lens, tree_mask, num_nodes: int, num_slots: int):
    """Return [bad lengths, bad table entries, mask rows with bits past N] as ints."""
    pt = np.asarray(page_table, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    mk = np.asarray(tree_mask).astype(np.uint32)
    B, max_kv = pt.shape
    N = int(num_nodes)
    bad_len = bad_slot = bad_mask = 0
    for b in range(B):
        raw = int(sl[b])
        if raw < N or raw > max_kv:
            bad_len += 1
        S = min(max(raw, N), max_kv)
        for p in range(S):
            v = int(pt[b, p])
            if v < 0 or v >= num_slots:
                bad_slot += 1
        for i in range(N):
            words = mk[b, i]
            past = False
            for w in range(len(words)):
                for bit in range(32):
                    if (int(words[w]) >> bit) & 1 and 32 * w + bit >= N:
                        past = True
            if past:
                bad_mask += 1
    return [bad_len, bad_slot, bad_mask]
