"""Seeded synthetic inputs for tree-verify MLA attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through its binding) and the CPU
oracle consume what it produces.

Workload shapes follow the pages' deployment: Kimi K2.6 MLA with a 576-wide
latent row (512 latent + 64 rope) kept in a page_size=1 pool and reached
through a per-token slot table ("The Architecture Detective", section "The
Context: A Bottleneck Confirmed"), a draft tree verified per decode step,
and 8 heads per tensor-parallel rank ("The Execution Phase", section "The
Optimization That Unlocked 3-6x Speedup").  Values are N(0,1) drawn in fp32
and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

D_QK = 576          # latent (512) + rope (64) columns per row
D_V = 512           # latent columns, the value part of a row
MAX_TREE = 64       # draft nodes per request (one 64-bit ancestor mask)
SM_SCALE = 1.0 / math.sqrt(192.0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1 << 16) -> np.ndarray:
    """N(0,1) bf16 bits of the given shape, drawn row-chunk by row-chunk."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1) if len(shape) > 1 else out.reshape(-1, 1)
    for a in range(0, flat.shape[0], chunk_rows):
        b = min(flat.shape[0], a + chunk_rows)
        flat[a:b] = bf16_bits(rng.standard_normal((b - a, flat.shape[1]), dtype=np.float32))
    return out


# --------------------------------------------------------------------------- trees
def chain_tree(T: int) -> np.ndarray:
    """parent[i] = i - 1: a chain of draft tokens (plain causal block)."""
    return (np.arange(T, dtype=np.int32) - 1).astype(np.int32)


def random_tree(rng: np.random.Generator, T: int, max_depth: int = 6) -> np.ndarray:
    """Random topological tree/forest: parent[i] uniform over {-1} and the
    earlier nodes whose depth still allows a child (depth <= max_depth)."""
    parent = np.empty(T, dtype=np.int32)
    depth = np.empty(T, dtype=np.int32)
    for i in range(T):
        cands = [-1] + [j for j in range(i) if depth[j] < max_depth]
        p = int(cands[int(rng.integers(len(cands)))])
        parent[i] = p
        depth[i] = 1 if p == -1 else depth[p] + 1
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    d = np.empty(len(parent), dtype=np.int32)
    for i, p in enumerate(parent):
        d[i] = 1 if p == -1 else d[p] + 1
    return d


# --------------------------------------------------------------------------- slot tables
def table_permutation(rng, num_slots: int, n: int) -> np.ndarray:
    """First n entries of a seeded permutation of the pool."""
    return rng.permutation(num_slots)[:n].astype(np.int32)


def table_scattered(rng, num_slots: int, n: int) -> np.ndarray:
    """n distinct slots drawn uniformly, in random order (fully scattered)."""
    return rng.choice(num_slots, size=n, replace=False).astype(np.int32)


def table_contiguous(start: int, n: int) -> np.ndarray:
    return np.arange(start, start + n, dtype=np.int32)


def table_runs_mixed(rng, num_slots: int, L: int, T: int, max_run: int = 64) -> np.ndarray:
    """Prefix: half the entries in runs of consecutive physical slots (run
    length uniform in 1..max_run, runs never overlap), half as single uniform
    free slots; the fragments are shuffled.  Draft slots: fresh free slots."""
    used = np.zeros(num_slots, dtype=bool)
    frags = []
    in_runs = L // 2
    placed = 0
    while placed < in_runs:
        ln = min(int(rng.integers(1, max_run + 1)), in_runs - placed)
        while True:
            s = int(rng.integers(0, num_slots - ln + 1))
            if not used[s:s + ln].any():
                break
        used[s:s + ln] = True
        frags.append(np.arange(s, s + ln, dtype=np.int32))
        placed += ln
    free = np.flatnonzero(~used)
    singles = rng.choice(free, size=L - in_runs + T, replace=False).astype(np.int32)
    for s in singles[:L - in_runs]:
        frags.append(np.array([s], dtype=np.int32))
    order = rng.permutation(len(frags))
    prefix = np.concatenate([frags[i] for i in order]) if frags else np.zeros(0, np.int32)
    return np.concatenate([prefix, singles[L - in_runs:]]).astype(np.int32)


def tables_interleaved(rng, num_slots: int, lengths, max_run: int = 64):
    """Fragmented allocation shared by several requests: the pool is cut into
    runs of consecutive slots (length uniform in 1..max_run), the runs are
    shuffled and handed out round-robin to the requests until each holds its
    length."""
    cuts = []
    s = 0
    while s < num_slots:
        ln = min(int(rng.integers(1, max_run + 1)), num_slots - s)
        cuts.append((s, ln))
        s += ln
    order = rng.permutation(len(cuts))
    need = list(int(x) for x in lengths)
    parts = [[] for _ in need]
    have = [0] * len(need)
    r = 0
    for idx in order:
        if all(h >= n for h, n in zip(have, need)):
            break
        while have[r] >= need[r]:
            r = (r + 1) % len(need)
        st, ln = cuts[idx]
        take = min(ln, need[r] - have[r])
        parts[r].append(np.arange(st, st + take, dtype=np.int32))
        have[r] += take
        r = (r + 1) % len(need)
    if any(h < n for h, n in zip(have, need)):
        raise ValueError("pool too small for the requested lengths")
    return [np.concatenate(p) for p in parts]


# --------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    num_heads: int
    num_tree: np.ndarray            # int32 [B]
    prefix_len: np.ndarray          # int32 [B]
    q: np.ndarray                   # uint16 [sum T, H, 576]
    kv_pool: np.ndarray             # uint16 [num_slots, 576]
    slot_table: np.ndarray          # int32 [sum (L + T)]
    slot_indptr: np.ndarray         # int32 [B + 1]
    parent: np.ndarray              # int32 [sum T], request-local
    sm_scale: float = SM_SCALE
    meta: dict = field(default_factory=dict)

    @property
    def num_requests(self) -> int:
        return int(self.num_tree.shape[0])

    @property
    def num_slots(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def total_rows(self) -> int:
        return int(self.num_tree.sum()) * self.num_heads

    @property
    def num_keys(self) -> int:
        return int((self.prefix_len.astype(np.int64) + self.num_tree).sum())

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: each latent row once per call (576 bf16)."""
        return self.num_keys * D_QK * 2


def make_workload(name, num_heads, num_tree, prefix_len, num_slots, *, seed, table="scattered",
                  tree="random", max_depth=6, max_run=64, q_override=None) -> Workload:
    """Build a seeded workload.  Seeds are split with SeedSequence into
    independent streams for (q, kv pool, slot table, tree)."""
    num_tree = np.asarray(num_tree, dtype=np.int32).reshape(-1)
    prefix_len = np.asarray(prefix_len, dtype=np.int32).reshape(-1)
    B = num_tree.shape[0]
    assert prefix_len.shape[0] == B
    if (num_tree < 1).any() or (num_tree > MAX_TREE).any():
        raise ValueError("num_tree must be in 1..64")
    ss_q, ss_kv, ss_tab, ss_tree = np.random.SeedSequence(seed).spawn(4)
    r_q, r_kv, r_tab, r_tree = (np.random.default_rng(s) for s in (ss_q, ss_kv, ss_tab, ss_tree))

    lengths = (prefix_len.astype(np.int64) + num_tree).tolist()
    if table == "permutation":
        assert B == 1
        tabs = [table_permutation(r_tab, num_slots, lengths[0])]
    elif table == "scattered":
        allt = table_scattered(r_tab, num_slots, int(sum(lengths)))
        tabs = np.split(allt, np.cumsum(lengths)[:-1])
    elif table == "runs_mixed":
        assert B == 1
        tabs = [table_runs_mixed(r_tab, num_slots, int(prefix_len[0]), int(num_tree[0]), max_run)]
    elif table == "interleaved":
        tabs = tables_interleaved(r_tab, num_slots, lengths, max_run)
    elif table == "contiguous":
        offs = np.concatenate([[0], np.cumsum(lengths)[:-1]])
        tabs = [table_contiguous(int(o), int(n)) for o, n in zip(offs, lengths)]
    else:
        raise ValueError(table)
    slot_table = np.concatenate(tabs).astype(np.int32)
    slot_indptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)

    if tree == "chain":
        parents = [chain_tree(int(t)) for t in num_tree]
    elif tree == "random":
        parents = [random_tree(r_tree, int(t), max_depth) for t in num_tree]
    elif tree == "star":
        parents = [np.full(int(t), -1, dtype=np.int32) for t in num_tree]
    else:
        raise ValueError(tree)
    parent = np.concatenate(parents).astype(np.int32)

    total_tree = int(num_tree.sum())
    q = normal_bf16(r_q, (total_tree, num_heads, D_QK)) if q_override is None else q_override
    kv_pool = normal_bf16(r_kv, (num_slots, D_QK))
    return Workload(name=name, num_heads=int(num_heads), num_tree=num_tree, prefix_len=prefix_len,
                    q=q, kv_pool=kv_pool, slot_table=slot_table, slot_indptr=slot_indptr,
                    parent=parent, meta=dict(seed=seed, table=table, tree=tree, num_slots=num_slots))


# The five workloads of the verify step, numbered 1..5 (seed = number).
CONFIGS = {
    1: dict(name="tiny_h8_t4chain_l256", num_heads=8, num_tree=[4], prefix_len=[256],
            num_slots=1024, table="permutation", tree="chain"),
    2: dict(name="tp_rank_h8_t16_l4096", num_heads=8, num_tree=[16], prefix_len=[4096],
            num_slots=262144, table="scattered", tree="random"),
    3: dict(name="tp_rank_h8_t16_l65536", num_heads=8, num_tree=[16], prefix_len=[65536],
            num_slots=262144, table="runs_mixed", tree="random"),
    4: dict(name="full_heads_h64_t16_l200000", num_heads=64, num_tree=[16], prefix_len=[200000],
            num_slots=262144, table="scattered", tree="random"),
    5: dict(name="ragged_b4_h16_t32", num_heads=16, num_tree=[32, 32, 32, 32],
            prefix_len=[1024, 16384, 65536, 131072], num_slots=524288, table="interleaved",
            tree="random"),
}


def make_config(idx: int, seed: int | None = None) -> Workload:
    c = dict(CONFIGS[idx])
    name = c.pop("name")
    return make_workload(name, seed=idx if seed is None else seed, **c)
