"""GPU draft-tree marshaling (verify_attn_build_tree) against the plain
reference oracle.tree, bit for bit, and end to end through the verify call."""
import numpy as np
import pytest
import torch

import speculative_tree_verify_mla_amd as va
from oracle import tree as ot
from speculative_tree_verify_mla_amd import inputs
from test_parity import DEV, Dev, _t, check, say
from test_tree_oracle import _golden

pytestmark = pytest.mark.gpu


def _raw_batch(num_tree, prefix, seed, slots=4096):
    """A workload whose trees are relabeled at random: returns (workload,
    raw_parent, raw_slot, q in raw order) with the draft table entries
    blanked out."""
    rng = np.random.default_rng(seed)
    wl = inputs.make_workload("mar", 4, num_tree, prefix, slots, seed=seed,
                              table="interleaved" if len(num_tree) > 1 else "scattered")
    raw_parent = np.empty_like(wl.parent)
    raw_slot = np.empty_like(wl.parent)
    q_raw = np.empty_like(wl.q)
    t0 = 0
    for r, T in enumerate(wl.num_tree):
        sigma = rng.permutation(T)
        base = int(wl.slot_indptr[r]) + int(wl.prefix_len[r])
        for g in range(T):
            pg = wl.parent[t0 + g]
            raw_parent[t0 + sigma[g]] = -1 if pg == -1 else sigma[pg]
            raw_slot[t0 + sigma[g]] = wl.slot_table[base + g]
            q_raw[t0 + sigma[g]] = wl.q[t0 + g]
        t0 += T
    return wl, raw_parent, raw_slot, q_raw


def _gpu_marshal(wl, raw_parent, raw_slot, table, device_prefix=None):
    plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
    tab = _t(table)
    pre = wl.prefix_len if device_prefix is None else np.asarray(device_prefix, np.int32)
    perm, parent, anc, status = va.verify_attn_build_tree(
        plan, _t(raw_parent), _t(raw_slot), _t(pre), _t(wl.slot_indptr), tab)
    torch.cuda.synchronize()
    return (perm.cpu().numpy(), parent.cpu().numpy(), anc.cpu().numpy().view(np.uint64),
            status.cpu().numpy().view(np.uint32), tab.cpu().numpy(), plan)


@pytest.mark.parametrize("num_tree,prefix", [([1], [10]), ([5], [0]), ([16], [300]),
                                             ([64], [1000]), ([3, 33, 1, 64], [5, 70, 0, 400])])
def test_marshaling_matches_the_reference(num_tree, prefix):
    wl, rp, rs, _ = _raw_batch(num_tree, prefix, seed=sum(num_tree))
    table = wl.slot_table.copy()
    for r in range(len(num_tree)):
        b = int(wl.slot_indptr[r]) + int(wl.prefix_len[r])
        table[b:b + num_tree[r]] = -7
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, table)
    got = _gpu_marshal(wl, rp, rs, table)
    say(f"  marshal T={num_tree} status={got[3].tolist()}")
    for name, a, b in zip(("perm", "parent", "anc", "status", "table"), got[:5], ref):
        np.testing.assert_array_equal(a, b, err_msg=name)
    # the same draft slots come back, in breadth-first order of the tree
    np.testing.assert_array_equal(np.sort(got[4]), np.sort(wl.slot_table))


def test_hand_worked_trees_on_the_gpu():
    cases = _golden()
    num_tree = [len(c["raw_parent"]) for c in cases]
    wl = inputs.make_workload("g", 1, num_tree, [2] * len(cases), 256, seed=3, table="interleaved")
    rp = np.concatenate([np.array(c["raw_parent"], np.int32) for c in cases])
    rs = np.arange(len(rp), dtype=np.int32) + 100
    perm, parent, anc, status, _, _ = _gpu_marshal(wl, rp, rs, wl.slot_table.copy())
    assert (status == 0).all()
    t0 = 0
    for c, T in zip(cases, num_tree):
        assert perm[t0:t0 + T].tolist() == c["perm"], c["name"]
        assert parent[t0:t0 + T].tolist() == c["parent"], c["name"]
        for i, pos in c["anc"].items():
            assert int(anc[t0 + i]) == sum(1 << k for k in pos), (c["name"], i)
        t0 += T


def test_bad_trees_are_flagged_per_request():
    wl, rp, rs, _ = _raw_batch([6, 6, 6], [20, 30, 40], seed=11)
    rp = rp.copy()
    rp[0:2] = [1, 0]                      # request 0: a cycle
    rp[6 + 3] = 6                         # request 1: parent out of range
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, wl.slot_table)
    got = _gpu_marshal(wl, rp, rs, wl.slot_table.copy())
    assert got[3][0] & ot.BAD_PARENT and got[3][1] & ot.BAD_PARENT and got[3][2] == 0
    for k in range(3):                    # request 2 is exact
        np.testing.assert_array_equal(got[k][12:], ref[k][12:])
    short = wl.slot_indptr.copy()
    short[3] -= 2                         # request 2's table range is 2 entries short
    wl2 = inputs.Workload(**{**wl.__dict__, "slot_indptr": short})
    got2 = _gpu_marshal(wl2, rp, rs, wl.slot_table.copy())
    assert got2[3][2] & ot.BAD_TABLE


def test_negative_device_prefix_writes_only_its_own_table_range():
    """A negative prefix length puts some of a request's draft entries below
    its table range: they are not written (the previous request's entries
    stay as they were) and the request is flagged."""
    wl, rp, rs, _ = _raw_batch([6, 8, 5], [20, 30, 40], seed=13)
    prefix = wl.prefix_len.copy()
    prefix[1] = -3                        # on the device only; the plan has the real bound
    before = wl.slot_table.copy()
    ref = ot.marshal(wl.num_tree, rp, rs, prefix, wl.slot_indptr, before)
    got = _gpu_marshal(wl, rp, rs, before, device_prefix=prefix)
    assert got[3][1] & ot.BAD_TABLE and got[3][0] == 0 and got[3][2] == 0
    np.testing.assert_array_equal(got[4], ref[4])
    # request 0's range holds exactly what a run with a valid request 1 writes
    ok = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, before)
    e0, e1 = int(wl.slot_indptr[0]), int(wl.slot_indptr[1])
    np.testing.assert_array_equal(got[4][e0:e1], ok[4][e0:e1])


def test_marshal_then_verify_in_one_graph():
    """Raw trees in, verify outputs out, all captured in one HIP graph of
    library calls (marshal, query permutation, verify); rows come out in
    verify order and match the oracle on the marshaled inputs."""
    wl, rp, rs, q_raw = _raw_batch([16, 9], [700, 1200], seed=21)
    d = Dev(wl)
    table = wl.slot_table.copy()
    for r in range(2):
        b = int(wl.slot_indptr[r]) + int(wl.prefix_len[r])
        table[b:b + int(wl.num_tree[r])] = -7
    d.table = _t(table)
    plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
    ws = va.workspace_for(plan, DEV)
    raw_p, raw_s = _t(rp), _t(rs)
    qr = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    qv = torch.empty_like(qr)
    H = wl.num_heads
    out = torch.empty((25, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((25, H), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            perm, parent, anc, status = va.verify_attn_build_tree(
                plan, raw_p, raw_s, d.prefix, d.indptr, d.table, stream=st)
            va.verify_attn_permute_rows(plan, perm, qr, qv, stream=st)
            va.verify_attn(qv, d.kv, d.table, d.indptr, d.prefix, parent, wl.sm_scale,
                           num_tree=wl.num_tree, prefix_len_host=wl.prefix_len, plan=plan,
                           workspace=ws, out=out, lse=lse, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, table)
    np.testing.assert_array_equal(d.table.cpu().numpy(), ref[4])
    perm_h = ref[0]
    q_v = np.concatenate([q_raw[:16][perm_h[:16]], q_raw[16:][perm_h[16:]]])
    wl_v = inputs.Workload(**{**wl.__dict__, "q": q_v, "parent": ref[1], "slot_table": ref[4]})
    check(wl_v, out, lse, what="marshal+verify graph")


def test_permute_rows_gathers_through_perm():
    """verify_attn_permute_rows against a host gather, bit for bit, for one and
    several requests; a perm entry outside the request's nodes gives zeros."""
    for num_tree in ([16], [3, 64, 1, 17]):
        H = 8
        plan = va.verify_attn_plan(H, [100] * len(num_tree), num_tree)
        n = int(plan.total_tree)
        rng = np.random.default_rng(len(num_tree))
        perm = np.concatenate([rng.permutation(t) for t in num_tree]).astype(np.int32)
        perm[1 if len(num_tree) == 1 else 5] = 70                  # outside [0, T_r)
        src = rng.standard_normal((n, H, 576)).astype(np.float32)
        src_b = torch.from_numpy(inputs.bf16_bits(src).view(np.int16)).to(DEV).view(torch.bfloat16)
        dst = va.verify_attn_permute_rows(plan, torch.from_numpy(perm).to(DEV), src_b)
        torch.cuda.synchronize()
        got = dst.view(torch.int16).cpu().numpy()
        want = np.zeros_like(got)
        srch = src_b.view(torch.int16).cpu().numpy()
        t0 = 0
        for t in num_tree:
            for i in range(t):
                j = int(perm[t0 + i])
                if 0 <= j < t:
                    want[t0 + i] = srch[t0 + j]
            t0 += t
        np.testing.assert_array_equal(got, want)


def _gather_rows(num_tree, perm, rows):
    """Host gather: row t0 + i of the result is rows[t0 + perm[t0 + i]]."""
    out = np.empty_like(rows)
    t0 = 0
    for t in num_tree:
        out[t0:t0 + t] = rows[t0:t0 + t][perm[t0:t0 + t]]
        t0 += t
    return out


@pytest.mark.parametrize("num_tree,prefix", [([1], [10]), ([16], [300]), ([64], [1000]),
                                             ([3, 33, 1, 64], [5, 70, 0, 400])])
def test_build_tree_rows_matches_the_reference(num_tree, prefix):
    """verify_attn_build_tree_rows (tree and query gather in one launch): the
    marshaled outputs against oracle.tree and the gathered query rows against
    a host gather through the oracle's perm, bit for bit."""
    wl, rp, rs, q_raw = _raw_batch(num_tree, prefix, seed=3 + sum(num_tree))
    table = wl.slot_table.copy()
    for r in range(len(num_tree)):
        b = int(wl.slot_indptr[r]) + int(wl.prefix_len[r])
        table[b:b + num_tree[r]] = -7
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, table)
    plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
    tab = _t(table)
    qr = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    perm, parent, anc, status, qv = va.verify_attn_build_tree_rows(
        plan, _t(rp), _t(rs), _t(wl.prefix_len), _t(wl.slot_indptr), tab, qr)
    torch.cuda.synchronize()
    got = (perm.cpu().numpy(), parent.cpu().numpy(), anc.cpu().numpy().view(np.uint64),
           status.cpu().numpy().view(np.uint32), tab.cpu().numpy())
    say(f"  build_tree_rows T={num_tree} status={got[3].tolist()}")
    assert (got[3] == 0).all()
    for k in range(5):
        np.testing.assert_array_equal(got[k], ref[k])
    want = _gather_rows(num_tree, ref[0], q_raw.view(np.int16))
    np.testing.assert_array_equal(qv.view(torch.int16).cpu().numpy(), want)


def test_build_tree_rows_flags_bad_requests_and_keeps_the_rest_exact():
    """A cycle and an out-of-range parent flag their requests as the two-call
    path does; the good request's outputs and rows stay exact, and a flagged
    request's rows are each one of its own raw rows or zeros."""
    wl, rp, rs, q_raw = _raw_batch([6, 6, 6], [20, 30, 40], seed=11)
    rp = rp.copy()
    rp[0:2] = [1, 0]                      # request 0: a cycle
    rp[6 + 3] = 6                         # request 1: parent out of range
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, wl.slot_table)
    plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
    tab = _t(wl.slot_table.copy())
    qr = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    perm, parent, anc, status, qv = va.verify_attn_build_tree_rows(
        plan, _t(rp), _t(rs), _t(wl.prefix_len), _t(wl.slot_indptr), tab, qr)
    torch.cuda.synchronize()
    st = status.cpu().numpy().view(np.uint32)
    assert st[0] & ot.BAD_PARENT and st[1] & ot.BAD_PARENT and st[2] == 0
    got = (perm.cpu().numpy(), parent.cpu().numpy(), anc.cpu().numpy().view(np.uint64))
    for k in range(3):
        np.testing.assert_array_equal(got[k][12:], ref[k][12:])
    rows = qv.view(torch.int16).cpu().numpy()
    qi = q_raw.view(np.int16)
    np.testing.assert_array_equal(rows[12:], _gather_rows([6], ref[0][12:], qi[12:]))
    for r in range(2):
        own = qi[6 * r:6 * r + 6]
        for i in range(6):
            row = rows[6 * r + i]
            assert not row.any() or any(np.array_equal(row, o) for o in own)


def test_build_tree_rows_then_verify_in_one_graph():
    """The one-launch marshaling and the verify call captured in one HIP graph,
    replayed three times with eager work and a synchronisation between the
    replays: every replay's output matches the oracle on the marshaled inputs."""
    wl, rp, rs, q_raw = _raw_batch([16, 9], [700, 1200], seed=23)
    d = Dev(wl)
    table = wl.slot_table.copy()
    for r in range(2):
        b = int(wl.slot_indptr[r]) + int(wl.prefix_len[r])
        table[b:b + int(wl.num_tree[r])] = -7
    d.table = _t(table)
    plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
    ws = va.workspace_for(plan, DEV)
    raw_p, raw_s = _t(rp), _t(rs)
    qr = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    qv = torch.empty_like(qr)
    H = wl.num_heads
    out = torch.empty((25, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((25, H), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            perm, parent, anc, status, _ = va.verify_attn_build_tree_rows(
                plan, raw_p, raw_s, d.prefix, d.indptr, d.table, qr, qv, stream=st)
            va.verify_attn(qv, d.kv, d.table, d.indptr, d.prefix, parent, wl.sm_scale,
                           num_tree=wl.num_tree, prefix_len_host=wl.prefix_len, plan=plan,
                           workspace=ws, out=out, lse=lse, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    ref = ot.marshal(wl.num_tree, rp, rs, wl.prefix_len, wl.slot_indptr, table)
    perm_h = ref[0]
    q_v = np.concatenate([q_raw[:16][perm_h[:16]], q_raw[16:][perm_h[16:]]])
    wl_v = inputs.Workload(**{**wl.__dict__, "q": q_v, "parent": ref[1], "slot_table": ref[4]})
    for rep in range(3):
        out.zero_()
        qv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == 0).all()
        np.testing.assert_array_equal(d.table.cpu().numpy(), ref[4])
        check(wl_v, out, lse, what=f"build_tree_rows+verify graph, replay {rep}")


def test_build_tree_rows_equals_the_two_calls_on_random_batches():
    """Random forests (1..6 requests of 1..64 nodes, any node order) and row
    widths whose last gather block is partial: the one-launch call writes
    exactly what verify_attn_build_tree + verify_attn_permute_rows write."""
    rng = np.random.default_rng(2024)
    for case in range(12):
        B = int(rng.integers(1, 7))
        num_tree = [int(x) for x in rng.integers(1, 65, size=B)]
        H = int(rng.choice([1, 3, 8]))
        prefix = [int(x) for x in rng.integers(0, 500, size=B)]
        raw_parent = []
        for t in num_tree:
            # parent of node j among nodes placed before it, then shuffled
            par = [-1] + [int(rng.integers(-1, j)) for j in range(1, t)]
            sigma = rng.permutation(t)
            rp = np.empty(t, np.int32)
            for j in range(t):
                rp[sigma[j]] = -1 if par[j] < 0 else sigma[par[j]]
            raw_parent.append(rp)
        raw_parent = np.concatenate(raw_parent).astype(np.int32)
        n = len(raw_parent)
        raw_slot = rng.integers(0, 1 << 20, size=n).astype(np.int32)
        indptr = np.concatenate([[0], np.cumsum(np.asarray(prefix) + np.asarray(num_tree) + 3)]).astype(np.int32)
        table = rng.integers(0, 1 << 20, size=int(indptr[-1])).astype(np.int32)
        plan = va.verify_attn_plan(H, prefix, num_tree)
        src = rng.standard_normal((n, H, 576)).astype(np.float32)
        src_b = torch.from_numpy(inputs.bf16_bits(src).view(np.int16)).to(DEV).view(torch.bfloat16)
        t1, t2 = _t(table), _t(table)
        a = va.verify_attn_build_tree(plan, _t(raw_parent), _t(raw_slot), _t(np.asarray(prefix, np.int32)),
                                      _t(indptr), t1)
        rows_a = va.verify_attn_permute_rows(plan, a[0], src_b)
        b = va.verify_attn_build_tree_rows(plan, _t(raw_parent), _t(raw_slot),
                                           _t(np.asarray(prefix, np.int32)), _t(indptr), t2, src_b)
        torch.cuda.synchronize()
        assert (a[3].cpu().numpy() == 0).all() and (b[3].cpu().numpy() == 0).all()
        for x, y in zip(a, b[:4]):
            assert torch.equal(x, y), case
        assert torch.equal(t1, t2), case
        assert torch.equal(rows_a.view(torch.int16), b[4].view(torch.int16)), case
