"""Host-side checks of libmk.so that need no GPU: the exported symbols, the
argument validation, and the host-built schedule (its structure and a
discrete-event proof that it cannot deadlock)."""
import ctypes
import os
import re
import subprocess

import pytest

from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mk.lib_path()):
        pytest.fail("libmk.so is not built (run python -m persistent_moe_amd.build)")
    return mk.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|void|const char\*)\s+(mk_\w+)\s*\(", src, re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(mk.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mk.lib_path()], capture_output=True, text=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for f in header_functions():
        assert f in syms, f
        assert hasattr(lib, f)


def test_strerror_names_every_code(lib):
    for code in range(0, -8, -1):
        assert mk.strerror(code) != "unknown error"


def test_task_descriptor_is_32_int32():
    assert ctypes.sizeof(mk.mk_task) == 128
    assert len(mk.OPCODES) == 16


def _cfg(model, B=1):
    return mk.make_config(model, B)


def test_workspace_size_validation(lib):
    assert mk.mk_workspace_size(_cfg(W.TINY_MOE), 8) > 0
    bad = _cfg(W.TINY_MOE)
    bad.head_dim = 96
    assert mk.mk_workspace_size(bad, 8) == 0
    bad = _cfg(W.TINY_MOE)
    bad.n_kv_heads = 3
    assert mk.mk_workspace_size(bad, 8) == 0
    assert mk.mk_workspace_size(_cfg(W.TINY_MOE), 0) == 0


def test_init_rejects_null_and_small_workspace(lib):
    cfg = _cfg(W.TINY_MOE)
    h = ctypes.c_void_p()
    w = mk.mk_weights()
    kv = mk.mk_kv_pool()
    rc = lib.mk_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), None, 0, 8, ctypes.byref(h))
    assert rc == mk.MK_E_INVAL
    rc = lib.mk_init(ctypes.byref(cfg), None, None, None, 0, 8, ctypes.byref(h))
    assert rc == mk.MK_E_INVAL
    # fake (never dereferenced) pointers: the size check comes before any device call
    L = cfg.n_layers
    arr = (mk.mk_layer_weights * L)()
    for l in range(L):
        for f in ("attn_norm", "w_qkv", "w_o", "w_router", "w_upgate", "w_down"):
            setattr(arr[l], f, 4096)
    w = mk.mk_weights(embed=4096, lm_head=4096, final_norm=4096, layers=arr)
    ptrs = (ctypes.c_void_p * L)(*([4096] * L))
    kv = mk.mk_kv_pool(k=ptrs, v=ptrs, num_pages=4)
    rc = lib.mk_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), ctypes.c_void_p(4096), 16, 8,
                     ctypes.byref(h))
    assert rc == mk.MK_E_NOMEM


def test_null_handle_calls_fail_cleanly(lib):
    assert lib.mk_build_schedule(None, 1, None) == mk.MK_E_INVAL
    assert lib.mk_decode_step(None, None, None, None, None, None, None) == mk.MK_E_INVAL
    smp = mk.make_sampling(0.7, 3, advance=True)
    assert lib.mk_decode_step_sample(None, None, None, None, None, None, ctypes.byref(smp), None, None) == mk.MK_E_INVAL
    assert lib.mk_get_status(None, None) == mk.MK_E_INVAL
    lib.mk_destroy(None)


def test_unsupported_shapes(lib):
    c = _cfg(W.DENSE_1B)
    c.max_batch = 4            # 4 x 8192 staged floats exceed the LDS staging area
    assert mk.mk_workspace_size(c, 8) == 0
    c = _cfg(W.TINY_MOE)
    c.max_batch = 9
    assert mk.mk_workspace_size(c, 8) == 0


def test_fp8_expert_config_rules(lib):
    assert mk.mk_workspace_size(_cfg(W.MOE_30B_FP8), 529) > 0
    assert mk.mk_workspace_size(_cfg(W.MOE_30B_FP8, 8), 529) > 0
    c = _cfg(W.MOE_30B)
    c.expert_fp8 = 2
    assert mk.mk_workspace_size(c, 8) == 0
    c = _cfg(W.DENSE_1B)
    c.expert_fp8 = 1                                                 # no experts to store
    assert mk.mk_workspace_size(c, 8) == 0
    c = _cfg(W.MOE_30B_FP8)
    c.expert_inter = 4096                                            # beyond two 1024-element chunks
    assert mk.mk_workspace_size(c, 8) == 0
    c = _cfg(W.MOE_30B_FP8)
    c.expert_inter = 760                                             # rows of whole 16-byte loads
    assert mk.mk_workspace_size(c, 8) == 0
    # FP8 experts without their row scales
    cfg = _cfg(W.TINY_MOE)
    cfg.expert_fp8 = 1
    L = cfg.n_layers
    arr = (mk.mk_layer_weights * L)()
    for l in range(L):
        for f in ("attn_norm", "w_qkv", "w_o", "w_router", "w_upgate", "w_down"):
            setattr(arr[l], f, 4096)
    w = mk.mk_weights(embed=4096, lm_head=4096, final_norm=4096, layers=arr)
    ptrs = (ctypes.c_void_p * L)(*([4096] * L))
    kv = mk.mk_kv_pool(k=ptrs, v=ptrs, num_pages=4)
    h = ctypes.c_void_p()
    rc = lib.mk_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), ctypes.c_void_p(4096), 1 << 30, 8,
                     ctypes.byref(h))
    assert rc == mk.MK_E_INVAL


def _plan(model, B, max_blocks, nw=256, order="tuned", split=0, opts=None):
    opts = opts if opts is not None else mk.make_opts(order, attn_split=split)
    return mk.mk_plan_schedule(_cfg(model, B), B, max_blocks, opts, nw)


@pytest.mark.parametrize("model,B,mb", [(W.TINY_MOE, 1, 5), (W.MOE_30B, 1, 529), (W.MOE_30B, 8, 1041),
                                        (W.DENSE_1B, 1, 264), (W.MOE_30B_SWA, 1, 16388)])
def test_plan_structure(lib, model, B, mb):
    tasks, nctr = _plan(model, B, mb)
    ops = [t.op for t in tasks]
    assert all(0 <= o < 16 for o in ops)
    L = model.n_layers
    norms = [t for t in tasks if t.op == 0]
    assert len(norms) == B * (L + 1 + (0 if model.parallel_block else L))   # one per sequence
    assert sorted({t.batch for t in norms}) == list(range(B))
    assert sum(1 for t in tasks if t.op == mk.OPCODES.index("LM_HEAD")) > 0
    lm = [t for t in tasks if t.op == mk.OPCODES.index("LM_HEAD")]
    assert lm[0].n0 == 0 and lm[-1].n1 == model.vocab
    assert all(a.n1 == b.n0 for a, b in zip(lm, lm[1:]))
    # every counter referenced lies inside the counter array
    for t in tasks:
        for c in (t.wait_ctr, t.signal_ctr, t.queue):
            assert -1 <= c < nctr
    # QKV tiles cover every rotation pair exactly once
    q = [t for t in tasks if t.op == 1 and t.layer == 0]
    pairs = (model.n_q_heads + 2 * model.n_kv_heads) * model.head_dim // 2
    assert q[0].n0 == 0 and q[-1].n1 == pairs and all(a.n1 == b.n0 for a, b in zip(q, q[1:]))


def test_static_tiles_dealt_round_robin(lib):
    # default placement, task k on workgroup k mod N: with 256 workgroups the
    # 256 QKV tiles of a layer of the 30B model land on 256 different workgroups
    tasks, _ = _plan(W.MOE_30B, 1, 529, order="interleaved")
    assert all(t.aux[16] == i % 256 and t.aux[17] == i for i, t in enumerate(tasks))
    idx = [i for i, t in enumerate(tasks) if t.op == 1 and t.layer == 3]
    assert len(idx) == 256
    assert len({i % 256 for i in idx}) == 256


def test_tuned_order_gives_router_tiles_their_own_workgroups(lib):
    tasks, _ = _plan(W.MOE_30B, 1, 529)
    assert all(t.aux[17] == i for i, t in enumerate(tasks))
    for l in (0, 7, 47):
        r = [t for t in tasks if mk.OPCODES[t.op] == "ROUTER_GEMM" and t.layer == l]
        q = [t for t in tasks if mk.OPCODES[t.op] == "QKV_PROJ" and t.layer == l]
        assert sorted(t.aux[16] for t in r) == list(range(8))
        wq = [t.aux[16] for t in q]
        assert len(set(wq)) == len(wq) and min(wq) >= 8 and max(wq) < 256
        # router tiles come before the QKV tiles in the list
        assert max(t.aux[17] for t in r) < min(t.aux[17] for t in q)


@pytest.mark.parametrize("model,B,mb,nw", [(W.MOE_30B, 1, 529, 256), (W.MOE_30B, 2, 40, 256),
                                           (W.MOE_30B_SWA, 1, 16388, 256), (W.TINY_MOE, 1, 5, 7),
                                           (W.MOE_30B, 1, 529, 200), (W.MOE_30B, 1, 529, 250),
                                           (W.MOE_30B, 1, 529, 128)])
def test_attention_owners_placement(lib, model, B, mb, nw):
    """Tuned order with a quarter to half of the grid's worth of attention
    splits: one ATTN_DRAIN claimer per split at the longest context, on
    distinct workgroups spread over the grid, each followed by its O-proj
    tile; the up-gate drain on every other workgroup; the down drain on all.
    Otherwise, and with MK_SCHED_SHARED_ATTN, every drain and one O-proj tile
    on every workgroup."""
    op = {n: i for i, n in enumerate(mk.OPCODES)}
    tasks, _ = _plan(model, B, mb, nw=nw)
    shared, _ = _plan(model, B, mb, nw=nw, opts=mk.make_opts(flags=mk.MK_SCHED_SHARED_ATTN))
    S = _plan_split(model, B, mb, nw, tasks)
    names = ("ATTN_DRAIN", "MOE_UPGATE_ACT_DRAIN", "O_PROJ", "MOE_DOWN_DRAIN")
    kinds = {op[n]: n for n in names}
    by = {}        # (layer, opcode name) -> tasks, in list order
    for ts, tag in ((tasks, ""), (shared, "shared:")):
        for t in ts:
            if t.op in kinds:
                by.setdefault((t.layer, tag + kinds[t.op]), []).append(t)
    for l in range(model.n_layers):
        vis = mb * 16
        if model.swa_window and model.swa_period and l % model.swa_period != model.swa_period - 1:
            vis = min(vis, model.swa_window)
        n_items = B * model.n_kv_heads * -(-vis // S)
        at, ug, oproj, dn = (by.get((l, n), []) for n in names)
        assert {t.aux[16] for t in by[(l, "shared:ATTN_DRAIN")]} == set(range(nw))
        assert {t.aux[16] for t in by[(l, "shared:MOE_UPGATE_ACT_DRAIN")]} == set(range(nw))
        assert {t.aux[16] for t in dn} == set(range(nw))
        if n_items > nw // 2 or n_items < nw // 4:   # too many or too few splits: shared
            assert len(at) == nw and len(ug) == nw
            continue
        owners = [t.aux[16] for t in at]
        assert len(at) == n_items and len(set(owners)) == n_items
        assert [t.n0 for t in at] == list(range(n_items)) and all(t.n1 == n_items for t in at)
        assert {t.aux[16] for t in ug} == set(range(nw)) - set(owners)
        # the O-proj tiles cover every output row of every group, on owners only
        assert {t.aux[16] for t in oproj} <= set(owners)
        for g in range(model.n_kv_heads):
            rows = sorted((t.n0, t.n1) for t in oproj if t.group == g)
            assert rows[0][0] == 0 and rows[-1][1] == model.d_model
            assert all(a[1] == b[0] for a, b in zip(rows, rows[1:]))
        # on each owner: attention, then its O-proj tile, then the down drain
        # (list order of one workgroup is builder order, aux[17])
        seq = {}
        for t in sorted(at + oproj + dn + ug, key=lambda t: t.aux[17]):
            seq.setdefault(t.aux[16], []).append(t.op)
        for w in owners:
            assert seq[w][0] == op["ATTN_DRAIN"] and seq[w][-1] == op["MOE_DOWN_DRAIN"]
            assert op["MOE_UPGATE_ACT_DRAIN"] not in seq[w]
        # spread: every XCD (workgroup mod 8) holds owners when there are at least 8
        if len(owners) >= 8 and nw % 8 == 0:
            assert {w % 8 for w in owners} == set(range(8))


def _plan_split(model, B, mb, nw, default_tasks):
    """The split length the builder chose: the explicit length whose plan
    equals the default one."""
    cfg = _cfg(model, B)
    want = [(t.op, t.aux[16], t.n0, t.n1) for t in default_tasks]
    for S in range(16, 4097, 16):
        try:
            a, _ = mk.mk_plan_schedule(cfg, B, mb, mk.make_opts(attn_split=S), nw)
        except Exception:
            continue
        if [(t.op, t.aux[16], t.n0, t.n1) for t in a] == want:
            return S
    raise AssertionError("split length not found")


def test_partitioned_order_places_branches_on_disjoint_sets(lib):
    # attention and O-proj on every 4th block of 8 workgroups (all 8 XCDs),
    # router and MoE projections on the rest; QKV and LM head on all
    opts = mk.make_opts("partitioned")
    tasks, _ = mk.mk_plan_schedule(mk.make_config(W.MOE_30B, 1), 1, 529, opts, 256)
    set_a = {w for w in range(256) if (w // 8) % 4 == 0}
    assert len(set_a) == 64 and {w % 8 for w in set_a} == set(range(8))
    where = {}
    for t in tasks:
        where.setdefault(mk.OPCODES[t.op], set()).add(t.aux[16])
    for op in ("ATTN_DRAIN", "O_PROJ", "ADD_RMSNORM"):
        assert where[op] <= set_a, op
    for op in ("ROUTER_GEMM", "MOE_UPGATE_ACT_DRAIN", "MOE_DOWN_DRAIN"):
        assert not (where[op] & set_a), op
    assert len(where["QKV_PROJ"]) == 256 and len(where["LM_HEAD"]) == 256
    # one attention claimer per attention workgroup and layer, combine fused
    a0 = [t for t in tasks if mk.OPCODES[t.op] == "ATTN_DRAIN" and t.layer == 0]
    assert len(a0) == 64 and all(t.flags & 32 and t.n1 == 64 for t in a0)
    assert "ATTN_COMBINE" not in where


def test_signal_counts_match_wait_targets(lib):
    # a static wait target must equal the number of tasks that signal it
    for model, B, mb in [(W.MOE_30B, 1, 529), (W.DENSE_1B, 1, 264), (W.TINY_MOE, 2, 6)]:
        tasks, _ = _plan(model, B, mb)
        sig = {}
        fused = {}
        G = model.n_q_heads // model.n_kv_heads
        for t in tasks:
            if t.signal_ctr >= 0:
                # a combine task adds its group's head count
                inc = G if t.op == mk.OPCODES.index("ATTN_COMBINE") else 1
                sig[t.signal_ctr] = sig.get(t.signal_ctr, 0) + inc
            if t.flags & 16:           # router tile with fused top-k: one ROUTE signal per layer
                fused[t.layer] = t.signal_ctr
        fused_comb = {t.layer for t in tasks if t.op == mk.OPCODES.index("ATTN_DRAIN") and t.flags & 32}
        for t in tasks:
            if t.op == mk.OPCODES.index("MOE_UPGATE_ACT_DRAIN"):
                route = t.wait_ctr
                if t.layer in fused:
                    sig[route] = 1
            if t.op == mk.OPCODES.index("O_PROJ") and t.layer in fused_comb:
                # fused combine: the combining splits of each sequence add the
                # group's head count in all
                sig[t.wait_ctr] = B * G
        for t in tasks:
            if t.wait_ctr >= 0 and t.wait_target > 0 and t.op not in (8, 13, 14):
                assert sig.get(t.wait_ctr, 0) == t.wait_target, (mk.OPCODES[t.op], t.layer)


@pytest.mark.parametrize("order", ["tuned", "interleaved", "attention_first", "partitioned", "tuned-separate-topk",
                                   "tuned-separate-combine", "partitioned-separate-combine", "tuned-static-moe",
                                   "tuned-separate-finalize", "tuned-static-attn", "attention_first-static-attn",
                                   "tuned-shared-attn"])
@pytest.mark.parametrize("case", [
    ("tiny", W.TINY_MOE, 1, 5, [65], [2, 2]),
    ("moe30b", W.MOE_30B, 1, 529, [8193], [8] * 48),
    ("moe30b-bs8", W.MOE_30B, 8, 1041, [512, 16384, 700, 3000, 9000, 1200, 15000, 2048], [52] * 48),
    ("moe30b-bs8-empty-slots", W.MOE_30B, 8, 1041, [0, 16384, 0, 3000, 0, 0, 0, 17], [16] * 48),
    ("dense", W.DENSE_1B, 1, 264, [4097], []),
])
def test_schedule_is_deadlock_free(lib, order, case):
    name, model, B, mb, sl, na = case
    flags = mk.MK_SCHED_SEPARATE_TOPK if order.endswith("separate-topk") else 0
    flags |= mk.MK_SCHED_SEPARATE_COMBINE if order.endswith("separate-combine") else 0
    flags |= mk.MK_SCHED_STATIC_MOE if order.endswith("static-moe") else 0
    if order.endswith("separate-finalize"):
        flags |= mk.MK_SCHED_SEPARATE_TOPK | mk.MK_SCHED_SEPARATE_FINALIZE
    flags |= mk.MK_SCHED_STATIC_ATTN if order.endswith("static-attn") else 0
    flags |= mk.MK_SCHED_SHARED_ATTN if order.endswith("shared-attn") else 0
    base = order.split("-")[0]
    opts = mk.make_opts(base, flags=flags)
    for nw in (256, 64, 7):
        rc, stuck = mk.mk_plan_simulate(_cfg(model, B), B, mb, opts, nw, sl, na)
        assert rc == mk.MK_OK, (name, nw, stuck)


def test_simulator_detects_a_blocked_schedule(lib):
    opts = mk.make_opts(flags=mk.MK_SCHED_UNREACHABLE_WAIT)
    rc, stuck = mk.mk_plan_simulate(_cfg(W.TINY_MOE, 1), 1, 5, opts, 4, [65], [2, 2])
    assert rc == mk.MK_E_STATE and stuck == 0
    rc = mk.mk_plan_simulate(_cfg(W.TINY_MOE, 1), 2, 5, mk.make_opts(), 4, [65, 65], [2, 2])[0]
    assert rc == mk.MK_E_INVAL   # batch above the configured maximum


def test_static_attention_and_separate_finalize_tasks(lib):
    """The static-attention schedule emits one ATTN_DECODE per (sequence, group,
    split) of the longest context and a combine per (sequence, group); the
    separate-finalize schedule emits ROUTE_FINALIZE after ROUTER_TOPK."""
    model, B, mb = W.MOE_30B, 2, 100      # 1600 keys at most
    tasks, _ = _plan(model, B, mb, opts=mk.make_opts(flags=mk.MK_SCHED_STATIC_ATTN))
    op = {n: i for i, n in enumerate(mk.OPCODES)}
    dec = [t for t in tasks if t.op == op["ATTN_DECODE"] and t.layer == 0]
    ns = max(t.split for t in dec) + 1
    assert len(dec) == B * model.n_kv_heads * ns
    assert {(t.batch, t.group) for t in dec} == {(b, g) for b in range(B) for g in range(model.n_kv_heads)}
    comb = [t for t in tasks if t.op == op["ATTN_COMBINE"] and t.layer == 0]
    assert len(comb) == B * model.n_kv_heads and all(t.wait_target == mk.MK_WAIT_SPLITS for t in comb)
    assert not any(t.op == op["ATTN_DRAIN"] for t in tasks)
    fl = mk.MK_SCHED_SEPARATE_TOPK | mk.MK_SCHED_SEPARATE_FINALIZE
    tasks, _ = _plan(model, B, mb, opts=mk.make_opts(flags=fl))
    top = [t for t in tasks if t.op == op["ROUTER_TOPK"] and t.layer == 3]
    fin = [t for t in tasks if t.op == op["ROUTE_FINALIZE"] and t.layer == 3]
    assert len(top) == 1 and len(fin) == 1 and not top[0].flags & 8
    assert fin[0].wait_ctr == top[0].signal_ctr == top[0].wait_ctr and fin[0].wait_target == top[0].wait_target + 1
