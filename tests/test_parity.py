"""GPU parity of the HIP verify path against the CPU fp64 oracle.

Every test calls the C ABI through the thin binding and compares element by
element with the oracle on the same seeded inputs.  Tolerances: max abs error
1e-2 on the bf16 output and 1e-3 on the fp32 LSE.  Gathers, permuted pools,
graph replays and repeated calls are compared bit for bit.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import speculative_tree_verify_mla_amd as va
from speculative_tree_verify_mla_amd import binding, inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _bf16(a):
    return _t(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


class Dev:
    """Device copies of a workload."""

    def __init__(self, wl, kv_pool=None):
        self.wl = wl
        self.q = _bf16(wl.q)
        self.kv = kv_pool if kv_pool is not None else _bf16(wl.kv_pool)
        self.table = _t(wl.slot_table)
        self.indptr = _t(wl.slot_indptr)
        self.prefix = _t(wl.prefix_len)
        self.parent = _t(wl.parent)


def run_gpu(wl, d=None, plan=None, prefix_host=None, rows=None):
    """rows: None (the planner's block size), 64 or 128 (forced)."""
    d = d or Dev(wl)
    plan = plan or va.verify_attn_plan(wl.num_heads, wl.prefix_len if prefix_host is None
                                       else prefix_host, wl.num_tree, rows=rows)
    if rows is not None:
        assert plan.groups_per_block == rows // 64
    ws = va.workspace_for(plan, DEV)
    out, lse = va.verify_attn(d.q, d.kv, d.table, d.indptr, d.prefix, d.parent, wl.sm_scale,
                              num_tree=wl.num_tree, prefix_len_host=wl.prefix_len, plan=plan,
                              workspace=ws)
    torch.cuda.synchronize()
    status = va.verify_attn_read_status(plan, ws)
    return out, lse, status, plan


def bf16_representation_error(ref):
    """|round_bf16(x) - x|: what any bf16 output must carry at the exact value x."""
    r32 = ref.astype(np.float32)
    rb = inputs.bf16_to_f32(inputs.bf16_bits(r32)).astype(np.float64)
    return np.abs(rb - ref)


# Where the exact value reaches 2, neighbouring bf16 values are 2^-6 or more
# apart: rounding alone may then miss it by 7.8e-3, and the kernel's own
# rounding (probabilities to bf16 for the value products, partials to fp16)
# adds up to a few 1e-3 on rows with few visible keys.  There the output is
# held to OUT_TOL beyond the rounding the exact value must carry; below 2
# (half spacing at most 3.9e-3) the plain bound applies.
REPR_FROM = 2.0


def check(wl, out, lse, rows=None, what="", ref=None):
    """Compare with the oracle, element by element.
    Output: |out - oracle| <= 1e-2 wherever |oracle| < 2; where |oracle| >= 2,
    |out - oracle| - (bf16 representation error of the oracle value) <= 1e-2.
    LSE: |lse - oracle| <= 1e-3 on every row.  ref: the oracle's (out, lse)
    for this workload, if already computed."""
    ref, ref_lse = ref if ref is not None else oracle.verify_attn_workload(wl, rows=rows)
    got = out.float().cpu().numpy().reshape(-1, 512).astype(np.float64)
    gl = lse.cpu().numpy().reshape(-1)
    ref = ref.reshape(-1, 512)
    ref_lse = ref_lse.reshape(-1)
    sel = np.arange(got.shape[0]) if rows is None else np.asarray(sorted(rows))
    r = ref[sel]
    diff = np.abs(got[sel] - r)
    small = np.abs(r) < REPR_FROM
    e_small = diff[small].max() if small.any() else 0.0
    beyond = diff - bf16_representation_error(r)
    e_large = beyond[~small].max() if (~small).any() else 0.0
    el = np.abs(gl[sel] - ref_lse[sel]).max()
    say(f"  {what} rows={len(sel)} max|out-oracle|={diff.max():.3e} (|oracle|<2: {e_small:.3e}; "
        f"beyond bf16 rounding at |oracle|>=2: {e_large:.3e}, {int((~small).sum())} elements) "
        f"max|lse-oracle|={el:.3e} max|oracle|={np.abs(r).max():.2f}")
    assert np.isfinite(got[sel]).all() and np.isfinite(gl[sel]).all()
    assert e_small <= OUT_TOL, e_small
    assert e_large <= OUT_TOL, e_large
    assert el <= LSE_TOL, el
    return diff.max(), el


# --------------------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_config_parity_all_rows(idx):
    """The five workloads, every output row against the oracle (the full-head
    and ragged ones take the oracle about 12 s and 6 s on 16 host cores).
    The full-head workload and the ragged batch get 128-row blocks from the
    planner; they are also run with 64-row blocks against the same oracle
    result."""
    wl = inputs.make_config(idx)
    say(f"config {idx} {wl.name}: H={wl.num_heads} T={wl.num_tree.tolist()} "
        f"L={wl.prefix_len.tolist()}")
    ref = oracle.verify_attn_workload(wl)
    for rows in ((None, 64) if idx in (4, 5) else (None,)):
        out, lse, status, plan = run_gpu(wl, rows=rows)
        assert status == 0
        say(f"  rows={64 * plan.groups_per_block} nsplit={plan.splits()} work={plan.total_work}")
        check(wl, out, lse, what=f"config {idx}", ref=ref)


# --------------------------------------------------------------------------- shapes and edges
EDGE = [
    # (H, T list, L list, tree)
    (1, [1], [0], "random"),
    (1, [1], [1], "random"),
    (3, [5], [1], "random"),
    (8, [16], [31], "random"),
    (8, [16], [32], "random"),
    (8, [16], [33], "random"),
    (5, [13], [100], "random"),
    (8, [4], [0], "chain"),
    (64, [64], [7], "random"),
    (16, [64], [1000], "star"),
    (2, [64], [300], "chain"),
    (7, [3, 17, 1, 64], [0, 45, 513, 2000], "random"),
]


EDGE_ROWS = [(c, None) for c in EDGE] + [(c, 128) for c in EDGE]


@pytest.mark.parametrize("case,rows", EDGE_ROWS,
                         ids=lambda c: f"H{c[0]}_T{c[1]}_L{c[2]}_{c[3]}" if isinstance(c, tuple)
                         else f"rows{c}")
def test_edge_shapes(case, rows):
    H, T, L, tree = case
    wl = inputs.make_workload("edge", H, T, L, 4096, seed=sum(L) + H, tree=tree,
                              table="interleaved" if len(T) > 1 else "scattered")
    say(f"edge H={H} T={T} L={L} {tree} rows={rows}")
    out, lse, status, _ = run_gpu(wl, rows=rows)
    assert status == 0
    check(wl, out, lse, what="edge")


@pytest.mark.parametrize("rows", [None, 128])
@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 64, 128])
def test_split_count_does_not_change_the_result(nsplit, rows, monkeypatch):
    wl = inputs.make_workload("ns", 8, [16], [4096], 16384, seed=3)
    monkeypatch.setenv("VA_NSPLIT", str(nsplit))
    say(f"VA_NSPLIT={nsplit} rows={rows}")
    out, lse, status, plan = run_gpu(wl, rows=rows)
    assert status == 0 and plan.nsplit[0] == nsplit
    check(wl, out, lse, what=f"nsplit {nsplit}")


@pytest.mark.parametrize("rows", [None, 128])
def test_split_of_draft_keys_only(rows, monkeypatch):
    """L = 1024, T = 64, 9 splits: the last split holds the 64 draft keys
    alone, and with a star tree node j sees only key L + j there (and all of
    the prefix elsewhere).  Every row still counts its own key."""
    monkeypatch.setenv("VA_NSPLIT", "9")
    wl = inputs.make_workload("draft_split", 4, [64], [1024], 4096, seed=71, tree="star")
    out, lse, status, plan = run_gpu(wl, rows=rows)
    assert status == 0 and plan.splits() == [9]
    check(wl, out, lse, what="draft-only split, star tree")


@pytest.mark.parametrize("rows", [None, 128])
def test_graph_bound_above_actual_prefix(rows):
    """Plan with an upper bound, run with a shorter device prefix length."""
    wl = inputs.make_workload("bound", 8, [16], [3000], 8192, seed=5)
    say("plan for L<=5000, run L=3000")
    out, lse, status, plan = run_gpu(wl, prefix_host=[5000], rows=rows)
    assert status == 0
    check(wl, out, lse, what="bound")


# --------------------------------------------------------------------------- coverage closed forms
@pytest.mark.parametrize("rows", [None, 128])
@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1000])
def test_zero_query_counts_every_visible_key(L, rows):
    """q = 0: lse = ln(number of visible keys) exactly; one key more or less
    moves it by >= 1e-3 at these lengths."""
    H, T = 4, 16
    wl = inputs.make_workload("q0", H, [T], [L], 4096, seed=100 + L,
                              q_override=np.zeros((T, H, 576), dtype=np.uint16))
    say(f"q=0 L={L} rows={rows}")
    out, lse, status, _ = run_gpu(wl, rows=rows)
    assert status == 0
    vis = oracle.tree_visibility(wl.parent)
    expect = np.log(L + vis.sum(1))
    got = lse.cpu().numpy()
    assert np.abs(got - expect[:, None]).max() <= LSE_TOL
    check(wl, out, lse, what="q=0")


def _needle(L, T, key, seed):
    H = 2
    wl = inputs.make_workload("needle", H, [T], [L], 4 * (L + T) + 64, seed=seed)
    wl.q = inputs.bf16_bits(np.full((T, H, 576), 0.5, dtype=np.float32))
    wl.kv_pool = wl.kv_pool.copy()
    wl.kv_pool[wl.slot_table[key]] = inputs.bf16_bits(
        np.linspace(-3.0, 3.0, 576, dtype=np.float32) * 0.25 + 4.0)
    return wl


@pytest.mark.parametrize("rows", [None, 128])
@pytest.mark.parametrize("nsplit", [1, 5])
def test_needle_at_tile_and_split_edges(nsplit, rows, monkeypatch):
    """A dominant key at every tile/split edge must reach every node's output."""
    L, T = 2000, 16
    monkeypatch.setenv("VA_NSPLIT", str(nsplit))
    per_split = -(-(L + T) // nsplit)
    chunk = -(-per_split // 32) * 32                       # split length in keys
    keys = sorted(set([0, 1, 30, 31, 32, 33, 63, 64, L - 1] +
                      [c + d for c in range(0, L, chunk) for d in (-1, 0) if 0 <= c + d < L]))
    for key in keys:
        wl = _needle(L, T, key, seed=7)
        out, lse, status, _ = run_gpu(wl, rows=rows)
        assert status == 0
        v = inputs.bf16_to_f32(wl.kv_pool[wl.slot_table[key]])[:512]
        err = np.abs(out.float().cpu().numpy() - v).max()
        say(f"  needle key={key} nsplit={nsplit} max|out-v|={err:.3e}")
        assert err <= OUT_TOL


@pytest.mark.parametrize("rows", [None, 128])
def test_needle_on_draft_nodes_respects_the_tree(rows):
    L, T = 700, 32
    base = inputs.make_workload("nd", 2, [T], [L], 4 * (L + T) + 64, seed=9)
    vis = oracle.tree_visibility(base.parent)
    for j in range(T):
        wl = _needle(L, T, L + j, seed=9)
        out, lse, status, _ = run_gpu(wl, rows=rows)
        assert status == 0
        v = inputs.bf16_to_f32(wl.kv_pool[wl.slot_table[L + j]])[:512]
        got = out.float().cpu().numpy()
        for i in range(T):
            near = np.abs(got[i] - v).max() <= OUT_TOL
            assert near == bool(vis[i, j]), (i, j)
        check(wl, out, lse, what=f"draft needle {j}")


def _rising(L, T, step, seed):
    """Prefix keys whose scores climb by about `step` log2 units from each
    64-key tile to the next: every row of tile j gets j * c added to its 64
    rope columns (q is 0.5 + 0.1 N(0, 1), so the score rises by about 32 c,
    a little differently for every query row), while the value columns stay
    N(0, 1)."""
    H = 2
    wl = inputs.make_workload("rising", H, [T], [L], 4 * (L + T) + 64, seed=seed)
    rng = np.random.default_rng(seed)
    wl.q = inputs.bf16_bits((0.5 + 0.1 * rng.standard_normal((T, H, 576))).astype(np.float32))
    log2_per_unit = 0.5 * 64 * wl.sm_scale / math.log(2.0)   # score rise per unit of c
    c = step / log2_per_unit
    pool = inputs.bf16_to_f32(wl.kv_pool)
    for k in range(L):
        pool[wl.slot_table[k], 512:] += np.float32(c * (k // 64))
    wl.kv_pool = inputs.bf16_bits(pool)
    return wl


@pytest.mark.parametrize("rows", [None, 128])
@pytest.mark.parametrize("nsplit", [1, 3])
def test_scores_rising_past_the_reference_on_every_tile(nsplit, rows, monkeypatch):
    """Tile maxima 100 log2 units apart over 12 tiles: each tile beats the
    previous one by more than the fixed-reference slack (64), so a split
    must find its exact max before its final pass.  The result is still the
    plain softmax attention of the oracle, with finite values everywhere.
    (128-row blocks step over 32-key tiles: every second one beats the
    previous by that much.)"""
    monkeypatch.setenv("VA_NSPLIT", str(nsplit))
    wl = _rising(L=64 * 12, T=4, step=100.0, seed=11)
    out, lse, status, plan = run_gpu(wl, rows=rows)
    assert status == 0
    check(wl, out, lse, what=f"rising scores nsplit={plan.splits()}")


# --------------------------------------------------------------------------- maximum sizes
@pytest.mark.parametrize("rows", [None, 128])
def test_maximum_request_count(rows):
    """VA_MAX_REQUESTS (64) requests of mixed tree sizes and prefixes in one
    call: every request's rows against the oracle."""
    rng = np.random.default_rng(64)
    B = binding.VA_MAX_REQUESTS
    T = rng.integers(1, 65, size=B).tolist()
    L = rng.integers(0, 1500, size=B).tolist()
    wl = inputs.make_workload("max_b", 2, T, L, 2 * (sum(T) + sum(L)) + 64, seed=64,
                              table="interleaved")
    out, lse, status, plan = run_gpu(wl, rows=rows)
    assert status == 0
    check(wl, out, lse, what=f"B={B} work={plan.total_work}")


def test_maximum_head_count_and_tree():
    """1024 heads x 64 draft nodes = 65536 query rows, every row against the
    oracle."""
    wl = inputs.make_workload("max_h", 1024, [64], [100], 4096, seed=65)
    out, lse, status, plan = run_gpu(wl)
    assert status == 0
    check(wl, out, lse, what=f"H=1024 T=64 work={plan.total_work}")


@pytest.mark.parametrize("rows", [None, 128])
def test_maximum_split_count(rows, monkeypatch):
    """VA_MAX_SPLITS (256) splits of one request: the reduce's largest
    instantiation merges them."""
    monkeypatch.setenv("VA_NSPLIT", str(binding.VA_MAX_SPLITS))
    wl = inputs.make_workload("max_s", 8, [16], [12000], 32768, seed=66)
    out, lse, status, plan = run_gpu(wl, rows=rows)
    assert status == 0
    assert plan.splits() == [binding.VA_MAX_SPLITS]
    check(wl, out, lse, what=f"nsplit={plan.splits()}")


def test_merge_with_four_quad_blocks_up_to_64_splits(monkeypatch):
    """One request with 32 row groups and 40 splits: the merge takes four
    quads per block (more one-quad blocks than one round of the CUs, at most
    64 splits).  Both block sizes against one oracle result."""
    monkeypatch.setenv("VA_NSPLIT", "40")
    wl = inputs.make_workload("quads", 64, [32], [10000], 16384, seed=67)
    ref = oracle.verify_attn_workload(wl)
    for rows in (64, 128):
        out, lse, status, plan = run_gpu(wl, rows=rows)
        assert status == 0 and plan.splits() == [40] and plan.num_groups[0] == 32
        check(wl, out, lse, what=f"40 splits, 32 row groups, rows={rows}", ref=ref)


# --------------------------------------------------------------------------- bit-exactness
@pytest.mark.parametrize("rows", [None, 128])
def test_permuted_pool_gives_identical_bits(rows):
    wl = inputs.make_workload("perm", 8, [16], [5000], 16384, seed=13)
    out, lse, _, _ = run_gpu(wl, rows=rows)
    pi = np.random.default_rng(1).permutation(wl.num_slots)
    pool2 = np.empty_like(wl.kv_pool)
    pool2[pi] = wl.kv_pool
    wl2 = inputs.Workload(**{**wl.__dict__, "kv_pool": pool2,
                             "slot_table": pi[wl.slot_table].astype(np.int32)})
    out2, lse2, _, _ = run_gpu(wl2, rows=rows)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


@pytest.mark.parametrize("rows", [None, 128])
def test_unused_slots_poisoned_with_nan_are_never_read(rows):
    wl = inputs.make_workload("poison", 8, [16], [3000], 8192, seed=17)
    out, lse, _, _ = run_gpu(wl, rows=rows)
    pool = wl.kv_pool.copy()
    unused = np.setdiff1d(np.arange(wl.num_slots), wl.slot_table)
    pool[unused] = 0x7FC0
    d = Dev(wl, kv_pool=_bf16(pool))
    out2, lse2, status, _ = run_gpu(wl, d=d, rows=rows)
    assert status == 0
    assert torch.isfinite(out2.float()).all()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


@pytest.mark.parametrize("rows", [None, 128])
def test_repeated_calls_are_bitwise_identical(rows):
    wl = inputs.make_workload("rep", 8, [16], [10000], 16384, seed=19)
    d = Dev(wl)
    a, la, _, plan = run_gpu(wl, d=d, rows=rows)
    for _ in range(3):
        b, lb, _, _ = run_gpu(wl, d=d, plan=plan)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))


@pytest.mark.parametrize("rows", [None, 128])
def test_padded_row_stride_matches_dense_pool(rows):
    wl = inputs.make_workload("stride", 4, [8], [900], 2048, seed=23)
    out, lse, _, _ = run_gpu(wl, rows=rows)
    wide = np.full((wl.num_slots, 640), 0x7FC0, dtype=np.uint16)
    wide[:, :576] = wl.kv_pool
    kv_wide = _bf16(wide)
    d = Dev(wl, kv_pool=kv_wide)
    assert kv_wide.stride(0) == 640
    out2, lse2, status, _ = run_gpu(wl, d=d, rows=rows)
    assert status == 0
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_gather_rows_is_bit_exact():
    rng = np.random.default_rng(29)
    pool = inputs.normal_bf16(rng, (5000, 576))
    table = rng.choice(5000, size=3001, replace=True).astype(np.int32)
    table[[5, 700]] = [-1, 5000]                              # invalid slots -> NaN rows
    dst = torch.empty((3001, 576), dtype=torch.bfloat16, device=DEV)
    va.verify_attn_gather_rows(_bf16(pool), _t(table), 3001, dst)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    ok = np.ones(3001, dtype=bool)
    ok[[5, 700]] = False
    np.testing.assert_array_equal(got[ok], pool[table[ok]])
    assert (got[~ok] == 0x7FC0).all()


@pytest.mark.parametrize("rows", [None, 128])
def test_graph_capture_replays_bit_exact_and_follows_device_lengths(rows):
    wl = inputs.make_workload("graph", 8, [16], [6000], 16384, seed=31)
    d = Dev(wl)
    plan = va.verify_attn_plan(8, [6000], [16], rows=rows)
    ws = va.workspace_for(plan, DEV)
    out = torch.empty((16, 8, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((16, 8), dtype=torch.float32, device=DEV)
    eager_o, eager_l = va.verify_attn(d.q, d.kv, d.table, d.indptr, d.prefix, d.parent,
                                      wl.sm_scale, num_tree=[16], prefix_len_host=[6000],
                                      plan=plan, workspace=ws)
    eager_o, eager_l = eager_o.clone(), eager_l.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            va.verify_attn(d.q, d.kv, d.table, d.indptr, d.prefix, d.parent, wl.sm_scale,
                           num_tree=[16], prefix_len_host=[6000], plan=plan, workspace=ws,
                           out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        torch.randn(1 << 20, device=DEV).sum().item()           # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(out.view(torch.int16), eager_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), eager_l.view(torch.int32))
    # shorter prefix through the device length only
    d.prefix.fill_(2500)
    g.replay()
    torch.cuda.synchronize()
    # the kernel now reads entries 0..2515 of the unchanged table: 2500 prefix
    # keys, then the draft nodes at entries 2500..2515
    wl3 = inputs.Workload(**{**wl.__dict__, "prefix_len": np.array([2500], np.int32),
                             "slot_table": wl.slot_table[:2516].copy(),
                             "slot_indptr": np.array([0, 2516], np.int32)})
    check(wl3, out, lse, what="replay L=2500")


# --------------------------------------------------------------------------- device-data errors
@pytest.mark.parametrize("rows", [None, 128])
def test_device_data_errors_poison_only_their_request(rows):
    wl = inputs.make_workload("err", 4, [8, 8], [300, 200], 4096, seed=37, table="interleaved")
    good_o, good_l, status, plan = run_gpu(wl, rows=rows)
    assert status == 0
    cases = []
    t = wl.slot_table.copy()
    t[10] = wl.num_slots + 5                                    # request 0, bad slot
    cases.append(("slot", dict(slot_table=t), 4))
    p = wl.parent.copy()
    p[3] = 5                                                    # request 0, parent >= i
    cases.append(("parent", dict(parent=p), 8))
    ind = wl.slot_indptr.copy()
    ind[1] = ind[1] - 5                                         # request 0 table too short
    cases.append(("short", dict(slot_indptr=ind), 2))
    for name, change, bit in cases:
        w2 = inputs.Workload(**{**wl.__dict__, **change})
        d = Dev(w2)
        o, l, status, _ = run_gpu(w2, d=d, plan=plan)
        say(f"  error case {name}: status={status}")
        assert status & bit
        of = o.float()
        assert torch.isnan(of[:8]).all() and torch.isnan(l[:8]).all()
        if name != "short":
            assert torch.equal(o[8:].view(torch.int16), good_o[8:].view(torch.int16))
    # device prefix above the planned bound
    d = Dev(wl)
    d.prefix[1] = 250
    o, l, status, _ = run_gpu(wl, d=d, plan=plan)
    assert status & 1
    assert torch.isnan(o[8:].float()).all()
    assert torch.equal(o[:8].view(torch.int16), good_o[:8].view(torch.int16))


@pytest.mark.parametrize("rows", [None, 128])
def test_single_request_table_offset_and_device_errors(rows):
    """A single request (the launches that take its values as preloaded
    kernel arguments): its table slice may start anywhere in the slot table,
    and a device prefix above the planned bound or a short slice still poison
    the rows and set the status bits."""
    wl = inputs.make_workload("one", 8, [16], [700], 4096, seed=41, table="interleaved")
    good_o, good_l, status, plan = run_gpu(wl, rows=rows)
    assert status == 0
    check(wl, good_o, good_l, what="offset 0")
    # the same slots behind 37 unrelated entries
    junk = np.arange(37, dtype=np.int32) % wl.num_slots
    off = inputs.Workload(**{**wl.__dict__, "slot_table": np.concatenate([junk, wl.slot_table]),
                             "slot_indptr": (wl.slot_indptr + 37).astype(np.int32)})
    o, l, status, _ = run_gpu(off, plan=plan)
    assert status == 0
    assert torch.equal(o.view(torch.int16), good_o.view(torch.int16))
    assert torch.equal(l.view(torch.int32), good_l.view(torch.int32))
    # device prefix above the planned bound
    d = Dev(wl)
    d.prefix.fill_(701)
    o, l, status, _ = run_gpu(wl, d=d, plan=plan)
    assert status & 1
    assert torch.isnan(o.float()).all() and torch.isnan(l).all()
    # a slice shorter than L + T
    short = inputs.Workload(**{**wl.__dict__,
                               "slot_indptr": np.array([0, 700 + 16 - 3], np.int32)})
    o, l, status, _ = run_gpu(short, plan=plan)
    assert status & 2
    assert torch.isnan(o.float()).all() and torch.isnan(l).all()
