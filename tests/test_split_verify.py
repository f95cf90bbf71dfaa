"""GPU parity of the split-verify decomposition.

VA_MODE_SPLIT_TREE runs a prefix kernel without any tree mask over the L
prefix keys and a small tree-block kernel over the T draft keys, joined by the
same log-sum-exp reduce ("The Architecture Detective", section "The Split
Verify Design").  It must match the CPU fp64 oracle to the same tolerances as
the fused mode (max abs error 1e-2 on the bf16 output, 1e-3 on the LSE), agree
with the fused mode, and keep the fused mode's bit-exactness properties
(graph replay, repeated calls).
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_tree_verify_mla_amd as va
from speculative_tree_verify_mla_amd import binding, inputs
from test_parity import (DEV, EDGE, LSE_TOL, OUT_TOL, Dev, _needle, _rising, check, run_gpu,
                         say)

pytestmark = pytest.mark.gpu


def split_plan(wl, prefix_host=None):
    return va.verify_attn_plan(wl.num_heads, wl.prefix_len if prefix_host is None else prefix_host,
                               wl.num_tree, split_tree=True)


def run_split(wl, d=None, prefix_host=None):
    plan = split_plan(wl, prefix_host)
    assert plan.mode == binding.VA_MODE_SPLIT_TREE
    return run_gpu(wl, d=d, plan=plan)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_split_config_parity_all_rows(idx):
    wl = inputs.make_config(idx)
    say(f"split config {idx} {wl.name}")
    out, lse, status, plan = run_split(wl)
    assert status == 0
    say(f"  nsplit={plan.splits()} (prefix splits + tree block) work={plan.total_work}")
    check(wl, out, lse, what=f"split config {idx}")


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"H{c[0]}_T{c[1]}_L{c[2]}_{c[3]}")
def test_split_edge_shapes(case):
    H, T, L, tree = case
    wl = inputs.make_workload("edge", H, T, L, 4096, seed=sum(L) + H, tree=tree,
                              table="interleaved" if len(T) > 1 else "scattered")
    say(f"split edge H={H} T={T} L={L} {tree}")
    out, lse, status, _ = run_split(wl)
    assert status == 0
    check(wl, out, lse, what="split edge")


def test_split_and_fused_modes_agree():
    wl = inputs.make_workload("ab", 8, [16], [9000], 16384, seed=41)
    d = Dev(wl)
    fo, fl, s1, _ = run_gpu(wl, d=d)
    so, sl, s2, _ = run_split(wl, d=d)
    assert s1 == 0 and s2 == 0
    do = (fo.float() - so.float()).abs().max().item()
    dl = (fl - sl).abs().max().item()
    say(f"  fused vs split: max|dout|={do:.3e} max|dlse|={dl:.3e}")
    assert do <= OUT_TOL and dl <= LSE_TOL


@pytest.mark.parametrize("nsplit", [1, 2, 7])
def test_split_prefix_split_count_does_not_change_the_result(nsplit, monkeypatch):
    wl = inputs.make_workload("ns", 8, [16], [4096], 16384, seed=3)
    monkeypatch.setenv("VA_NSPLIT", str(nsplit))
    out, lse, status, plan = run_split(wl)
    assert status == 0 and plan.nsplit[0] == nsplit + 1
    check(wl, out, lse, what=f"split prefix nsplit {nsplit}")


@pytest.mark.parametrize("L", [0, 1, 32, 33, 257, 1000])
def test_split_zero_query_counts_every_visible_key(L):
    H, T = 4, 16
    wl = inputs.make_workload("q0", H, [T], [L], 4096, seed=100 + L,
                              q_override=np.zeros((T, H, 576), dtype=np.uint16))
    out, lse, status, _ = run_split(wl)
    assert status == 0
    vis = oracle.tree_visibility(wl.parent)
    expect = np.log(L + vis.sum(1))
    assert np.abs(lse.cpu().numpy() - expect[:, None]).max() <= LSE_TOL
    check(wl, out, lse, what=f"split q=0 L={L}")


def test_split_needles_at_the_prefix_tree_seam():
    """Dominant keys at the last prefix key (prefix kernel) and on the draft
    nodes (tree kernel): the prefix needle reaches every node, a draft needle
    only the node and its descendants."""
    L, T = 700, 32
    base = inputs.make_workload("nd", 2, [T], [L], 4 * (L + T) + 64, seed=9)
    vis = oracle.tree_visibility(base.parent)
    for key in [L - 1, L, L + 1, L + T - 1]:
        wl = _needle(L, T, key, seed=9)
        out, lse, status, _ = run_split(wl)
        assert status == 0
        v = inputs.bf16_to_f32(wl.kv_pool[wl.slot_table[key]])[:512]
        got = out.float().cpu().numpy()
        for i in range(T):
            near = np.abs(got[i] - v).max() <= OUT_TOL
            assert near == (key < L or bool(vis[i, key - L])), (key, i)
        say(f"  split needle key={key} ok")


def test_split_scores_rising_past_the_reference_on_every_tile(monkeypatch):
    """The prefix kernel's splits see tile maxima 100 log2 units apart (more
    than the fixed-reference slack): the result is still the oracle's."""
    monkeypatch.setenv("VA_NSPLIT", "3")
    wl = _rising(L=64 * 12, T=4, step=100.0, seed=12)
    out, lse, status, plan = run_split(wl)
    assert status == 0
    check(wl, out, lse, what=f"split rising scores nsplit={plan.splits()}")


def test_split_graph_capture_replays_bit_exact_and_follows_device_lengths():
    wl = inputs.make_workload("graph", 8, [16], [6000], 16384, seed=31)
    d = Dev(wl)
    plan = va.verify_attn_plan(8, [6000], [16], split_tree=True)
    ws = va.workspace_for(plan, DEV)
    out = torch.empty((16, 8, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((16, 8), dtype=torch.float32, device=DEV)
    kw = dict(num_tree=[16], prefix_len_host=[6000], plan=plan, workspace=ws)
    eo, el = va.verify_attn(d.q, d.kv, d.table, d.indptr, d.prefix, d.parent, wl.sm_scale, **kw)
    eo, el = eo.clone(), el.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            va.verify_attn(d.q, d.kv, d.table, d.indptr, d.prefix, d.parent, wl.sm_scale,
                           out=out, lse=lse, **kw)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.zero_()
        torch.randn(1 << 20, device=DEV).sum().item()
        g.replay()
        torch.cuda.synchronize()
        say(f"  split replay {rep}")
        assert torch.equal(out.view(torch.int16), eo.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), el.view(torch.int32))
    check(wl, out, lse, what="split replay")
    d.prefix.fill_(2500)
    g.replay()
    torch.cuda.synchronize()
    wl3 = inputs.Workload(**{**wl.__dict__, "prefix_len": np.array([2500], np.int32),
                             "slot_table": wl.slot_table[:2516].copy(),
                             "slot_indptr": np.array([0, 2516], np.int32)})
    check(wl3, out, lse, what="split replay L=2500")


def test_split_device_data_errors_poison_only_their_request():
    wl = inputs.make_workload("err", 4, [8, 8], [300, 200], 4096, seed=37, table="interleaved")
    good_o, good_l, status, plan = run_split(wl)
    assert status == 0
    p = wl.parent.copy()
    p[3] = 5                                                    # request 0, parent >= i
    t = wl.slot_table.copy()
    t[10] = wl.num_slots + 5                                    # request 0, bad prefix slot
    t2 = wl.slot_table.copy()
    t2[300 + 2] = -3                                            # request 0, bad draft slot
    for name, change, bit in (("parent", dict(parent=p), 8), ("slot", dict(slot_table=t), 4),
                              ("draft slot", dict(slot_table=t2), 4)):
        w2 = inputs.Workload(**{**wl.__dict__, **change})
        o, l, status, _ = run_gpu(w2, d=Dev(w2), plan=plan)
        say(f"  split error case {name}: status={status}")
        assert status & bit
        assert torch.isnan(o[:8].float()).all() and torch.isnan(l[:8]).all()
        assert torch.equal(o[8:].view(torch.int16), good_o[8:].view(torch.int16))
