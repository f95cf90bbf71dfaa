"""GPU slot compaction (verify_attn_compact) against the plain reference
oracle.compact, bit for bit: the rewritten table, every pool row and the
count of copied rows."""
import numpy as np
import pytest
import torch

import speculative_tree_verify_mla_amd as va
from oracle import compact as oc
from speculative_tree_verify_mla_amd import inputs
from test_parity import DEV, Dev, _bf16, _t, run_gpu, say

pytestmark = pytest.mark.gpu


def _pool_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run_compact(table, pool, dst, budget):
    """GPU compaction on device copies; returns (table, pool, copied) on the host."""
    tab = _t(np.asarray(table, np.int32))
    kv = _bf16(pool)
    copied = va.verify_attn_compact(kv, tab, dst, budget)
    torch.cuda.synchronize()
    return tab.cpu().numpy(), _pool_u16(kv), int(copied.item())


def _check(table, pool, dst, budget, what):
    t_ref, p_ref, c_ref = oc.compact(table, pool, dst, budget)
    t, p, c = _run_compact(table, pool, dst, budget)
    say(f"  {what}: n={len(table)} budget={budget} copied={c} (oracle {c_ref}) "
        f"runs {oc.runs(table)} -> {oc.runs(t)}")
    assert c == c_ref
    np.testing.assert_array_equal(t, t_ref)
    assert np.array_equal(p, p_ref)


@pytest.mark.parametrize("n,budget", [(0, 5), (1, 1), (700, 0), (700, 1), (1025, 1000),
                                      (3000, 2500), (3000, 100000)])
def test_compaction_matches_the_reference(n, budget):
    rng = np.random.default_rng(n + budget)
    slots = 8192
    pool = inputs.normal_bf16(rng, (slots + n, 576))
    table = rng.choice(slots, size=n, replace=False).astype(np.int32)
    _check(table, pool, slots, budget, "random table")


def test_rows_already_in_place_are_skipped():
    rng = np.random.default_rng(2)
    n, dst = 2500, 6000
    pool = inputs.normal_bf16(rng, (dst + n, 576))
    table = rng.choice(dst, size=n, replace=False).astype(np.int32)
    inplace = rng.choice(n, size=900, replace=False)
    table[inplace] = dst + inplace
    for budget in (0, 37, 1200, n):
        _check(table, pool, dst, budget, "partly in place")


def test_long_request_with_runs_and_scatter():
    """The 65k-prefix workload's table (half runs, half scattered slots)."""
    wl = inputs.make_config(3)
    n = int(wl.slot_indptr[1])
    pool = np.concatenate([wl.kv_pool, np.zeros((n, 576), np.uint16)])
    for budget in (4096, n):
        _check(wl.slot_table, pool, wl.num_slots, budget, "65k request")


def test_precondition_failures_change_nothing():
    rng = np.random.default_rng(4)
    n, dst = 1500, 3000
    pool = inputs.normal_bf16(rng, (dst + n, 576))
    table = rng.choice(dst, size=n, replace=False).astype(np.int32)
    bad = table.copy()
    bad[700] = dst + n + 1000000                           # outside the pool
    occ = table.copy()
    occ[10] = dst + 11                                     # inside the run, wrong place
    both = bad.copy()
    both[10] = dst + 11
    for tb, code in ((bad, -1), (occ, -2), (both, -3)):
        t, p, c = _run_compact(tb, pool, dst, n)
        say(f"  precondition case: copied={c}")
        assert c == code
        np.testing.assert_array_equal(t, tb)
        assert np.array_equal(p, pool)


def test_verify_output_is_bitwise_unchanged_by_compaction():
    wl = inputs.make_workload("cmpv", 8, [16], [5000], 16384, seed=61, table="runs_mixed")
    n = int(wl.slot_indptr[1])
    d = Dev(wl)
    before_o, before_l, st, plan = run_gpu(wl, d=d)
    assert st == 0
    pool = torch.cat([d.kv, torch.zeros((n, 576), dtype=torch.bfloat16, device=DEV)])
    d.kv = pool
    copied = va.verify_attn_compact(pool, d.table, wl.num_slots, n)
    torch.cuda.synchronize()
    assert int(copied.item()) == n
    assert torch.equal(d.table.cpu(), torch.arange(wl.num_slots, wl.num_slots + n, dtype=torch.int32))
    after_o, after_l, st, _ = run_gpu(wl, d=d, plan=plan)
    assert st == 0
    assert torch.equal(before_o.view(torch.int16), after_o.view(torch.int16))
    assert torch.equal(before_l.view(torch.int32), after_l.view(torch.int32))


def test_compaction_in_a_graph_replays():
    rng = np.random.default_rng(6)
    n, dst = 2000, 5000
    pool = inputs.normal_bf16(rng, (dst + n, 576))
    table = rng.choice(dst, size=n, replace=False).astype(np.int32)
    t_ref, p_ref, c_ref = oc.compact(table, pool, dst, 1500)
    tab = _t(table)
    kv = _bf16(pool)
    ws = torch.empty(int(va.load_library().verify_attn_compact_workspace_bytes(n, 1500)),
                     dtype=torch.uint8, device=DEV)
    copied = torch.empty(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            va.verify_attn_compact(kv, tab, dst, 1500, workspace=ws, copied=copied)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    assert int(copied.item()) == c_ref == 1500
    np.testing.assert_array_equal(tab.cpu().numpy(), t_ref)
    assert np.array_equal(_pool_u16(kv), p_ref)
    # the second replay moves the remaining 500 rows
    t2, p2, c2 = oc.compact(t_ref, p_ref, dst, 1500)
    g.replay()
    torch.cuda.synchronize()
    assert int(copied.item()) == c2 == 500
    np.testing.assert_array_equal(tab.cpu().numpy(), t2)
    assert np.array_equal(_pool_u16(kv), p2)


def test_table_over_a_million_entries_uses_the_scan_pass():
    """More than 1024 count blocks (n > 2^20): the separate scan pass, with its
    carry across chunks of 1024 counts, selects the rows.  Slots come from a
    small range (duplicates are separate keys) so the pool stays ~1.2 GB."""
    rng = np.random.default_rng(9)
    n, src_slots = (1 << 20) + 1500, 4096
    pool = np.zeros((src_slots + n, 576), np.uint16)
    pool[:src_slots] = inputs.normal_bf16(rng, (src_slots, 576))
    table = rng.integers(0, src_slots, size=n).astype(np.int32)
    for budget in (5000, 0):
        _check(table, pool, src_slots, budget, "n > 2^20")
