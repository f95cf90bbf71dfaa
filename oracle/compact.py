"""Plain reference of the Tier 1 slot compaction of one request.

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests and the
benchmark call it; the product never imports it.

Source: "The Execution Phase: From Plan to 3-6x Decode Speedup on Blackwell
Consumer GPUs", section "Tier 0 KV Defragmentation" (the next tier is live
relocation of a request's fragmented KV slots under a copy budget), and "The
Architecture Detective", section "Deconstructing the K/V Defrag Hypothesis"
(relocating a request's KV entries to contiguous slots).  The pages fix no
policy; the one written out here, step by step in plain Python, is:

  logical position k belongs at slot dst_begin + k of a free run the caller
  reserved; walking k upward, each row not yet at its place is copied there
  and its table entry rewritten, until `budget` rows have been copied; rows
  already in place are skipped and do not count.

Preconditions: every slot lies in the pool, and no slot lies inside the run
except at its own place.  On a violation nothing is changed and the result is
minus the OR of the violated bits (1: slot outside the pool, 2: slot inside
the run at another place).
"""
from __future__ import annotations

import numpy as np

BAD_SLOT = 1
RUN_OCCUPIED = 2


def compact(table, pool, dst_begin, budget):
    """Return (new_table, new_pool, copied).  Inputs are not modified."""
    table = np.asarray(table, dtype=np.int64)
    n = len(table)
    num_slots = pool.shape[0]
    if dst_begin < 0 or dst_begin + n > num_slots or budget < 0:
        raise ValueError("run outside the pool or negative budget")
    bits = 0
    for k in range(n):
        s = int(table[k])
        if s < 0 or s >= num_slots:
            bits |= BAD_SLOT
        if dst_begin <= s < dst_begin + n and s != dst_begin + k:
            bits |= RUN_OCCUPIED
    new_table = table.copy()
    new_pool = pool.copy()
    if bits:
        return new_table.astype(np.int32), new_pool, -bits
    copied = 0
    for k in range(n):
        if copied == budget:
            break
        s = int(table[k])
        d = dst_begin + k
        if s == d:
            continue
        new_pool[d, :576] = pool[s, :576]
        new_table[k] = d
        copied += 1
    return new_table.astype(np.int32), new_pool, copied


def runs(table):
    """Number of maximal runs of consecutive slots (1 for a contiguous table)."""
    t = np.asarray(table, dtype=np.int64)
    if len(t) == 0:
        return 0
    return 1 + int(np.count_nonzero(t[1:] != t[:-1] + 1))
