"""Parity of the HIP decode path (through the C ABI) with the CPU oracle.

Small and reduced workloads run every step against the oracle; the full-size
30B / 3.3B-active model is checked on its first decode step at full size, in
the launch configuration bench.py times.
"""
import os

import numpy as np
import pytest
import torch

from oracle import decode as O
from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W
from tests.parity import Report, compare_step, run_teacher_forced, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu_available):
    mk.load()
    yield


def _engine(wl, **kw):
    from persistent_moe_amd.runner import DecodeEngine
    say("engine", wl.name, "B", wl.batch, kw)
    return DecodeEngine(wl, **kw)


# reduced shapes: the real head / expert geometry, fewer layers and a small vocab
MOE_SMALL = W.ModelConfig(name="moe30b-shape-2l", n_layers=2, d_model=2048, n_q_heads=32, n_kv_heads=4,
                          head_dim=128, vocab=4096, n_experts=128, top_k=8, expert_inter=768)
DENSE_SMALL = W.ModelConfig(name="dense1b-shape-2l", n_layers=2, d_model=2048, n_q_heads=32, n_kv_heads=8,
                            head_dim=64, vocab=2048, ffn_inter=8192, tied_embeddings=True,
                            parallel_block=False)
SWA_SMALL = W.ModelConfig(name="moe30b-swa-4l", n_layers=4, d_model=2048, n_q_heads=32, n_kv_heads=4,
                          head_dim=128, vocab=2048, n_experts=128, top_k=8, expert_inter=768,
                          swa_window=160, swa_period=4)


def test_tiny_moe_teacher_forced_all_steps():
    wl = W.WORKLOADS["tiny"]
    eng = _engine(wl)
    rep = run_teacher_forced(eng, wl.steps)
    rep.check()
    assert rep.compared == wl.steps


def test_moe30b_shape_ragged_context():
    # 333 cached tokens: the last page and the last attention split are partial
    wl = W.Workload("moe30b-shape-ctx333", MOE_SMALL, batch=1, ctx="fixed:333", steps=3, seed=11)
    eng = _engine(wl)
    run_teacher_forced(eng, 3).check()


def test_moe30b_shape_attention_owners():
    """2-layer 30B shape at 8,000 cached tokens, one row: the attention splits
    number between a quarter and half of the grid, so the default schedule
    gives them to attention owners, puts the O-proj tiles on the owners and
    sizes the up-gate and down items for the other workgroups."""
    wl = W.Workload("moe30b-shape-owners-ctx8000", MOE_SMALL, batch=1, ctx="fixed:8000", steps=3, seed=17)
    eng = _engine(wl)
    nw = torch.cuda.get_device_properties(0).multi_processor_count
    tasks, _ = mk.mk_plan_schedule(eng.mkcfg, 1, eng.max_blocks, eng.opts, nw)
    n_attn = sum(1 for t in tasks if t.layer == 0 and mk.OPCODES[t.op] == "ATTN_DRAIN")
    say("attention owners", n_attn, "of", nw)
    assert nw // 4 <= n_attn <= nw // 2
    run_teacher_forced(eng, 3).check()


def test_dense1b_shape_sequential_block():
    wl = W.Workload("dense1b-shape-ctx200", DENSE_SMALL, batch=1, ctx="fixed:200", steps=3, seed=12)
    eng = _engine(wl)
    run_teacher_forced(eng, 3).check()


def test_moe30b_shape_bs8_ragged_with_swap():
    wl = W.Workload("moe30b-shape-bs8", MOE_SMALL, batch=8, ctx="loguniform:20:700", steps=4, seed=13,
                    swap_every=2)
    eng = _engine(wl)
    rep = run_teacher_forced(eng, 4)
    rep.check()
    assert rep.rows == 32


@pytest.mark.parametrize("batch,n_wg", [(8, 12), (8, 40), (1, 16)])
def test_few_workgroups(batch, n_wg):
    # few workgroups: many attention splits and MoE items per claimer, and the
    # shared combine capped below one share per head (n_wg 12 and 40 at 8
    # sequences x 4 KV groups: 1 and 2 shares; 16 at one sequence: 4 shares
    # of 2 heads), so the spinning shares and the cap run on the device
    wl = W.Workload(f"moe30b-shape-b{batch}-{n_wg}wg", MOE_SMALL, batch=batch, ctx="loguniform:200:900",
                    steps=2, seed=17 + n_wg)
    eng = _engine(wl, opts=mk.make_opts(n_workgroups=n_wg))
    run_teacher_forced(eng, 2).check()


@pytest.mark.parametrize("batch,ug,dn", [(8, 100, 200), (1, 7, 300)])
def test_moe_tile_size_options(batch, ug, dn):
    # explicit MoE item sizes with ragged last tiles (768 = 7 x 100 + 68 or
    # 109 x 7 + 5 pairs; 2048 = 10 x 200 + 48 or 6 x 300 + 248 rows)
    wl = W.Workload(f"moe30b-shape-b{batch}-tiles", MOE_SMALL, batch=batch, ctx="loguniform:30:400",
                    steps=2, seed=41 + batch)
    eng = _engine(wl, opts=mk.make_opts(moe_ug_pairs=ug, moe_dn_rows=dn))
    run_teacher_forced(eng, 2).check()


def test_sliding_window_layers():
    wl = W.Workload("moe30b-swa-ctx300", SWA_SMALL, batch=1, ctx="fixed:300", steps=2, seed=14)
    eng = _engine(wl)
    run_teacher_forced(eng, 2).check()


def test_empty_slots_are_skipped():
    wl = W.Workload("tiny-bs4", W.TINY_MOE, batch=4, ctx="fixed:40", steps=1, seed=15)
    eng = _engine(wl)
    Wo = O.Weights(wl)
    t, pos, sl = eng.step_inputs()
    sl[1] = 0
    sl[3] = 0
    logits = eng.decode(inputs=(t, pos, sl))
    assert eng.status().code == 0
    lg = logits.cpu()
    assert torch.count_nonzero(lg[1]) == 0 and torch.count_nonzero(lg[3]) == 0
    rep = Report()
    res = [O.decode_one(wl, Wo, O.new_sequence(eng.slot_seq[b].seq_id, 40), eng.slot_tok[b]) for b in range(4)]
    compare_step(eng, res, logits, rep, [0, 2], check_taps=False)
    rep.check()


def test_determinism_same_inputs_same_bits():
    wl = W.Workload("moe30b-shape-det", MOE_SMALL, batch=2, ctx="fixed:100", steps=2, seed=16)
    eng = _engine(wl)
    inp = eng.step_inputs()
    a = eng.decode(inputs=inp).clone()
    assert eng.status().code == 0
    b = eng.decode(inputs=inp).clone()       # same inputs again (rewrites the same KV slot)
    assert eng.status().code == 0
    assert torch.equal(a, b)


# Every schedule the builder offers, each checked against the oracle
# (teacher-forced, two steps) and, on its first step, bit for bit against the
# tuned schedule: the same tiles in other placements, orders, task splits or
# launches must give the same bits (the split length is the minimum for these
# contexts in every order, so the attention partials are the same).
SCHEDULES = [
    ("tuned", {}),
    ("interleaved", dict(wave_order="interleaved")),
    ("attention_first", dict(wave_order="attention_first")),
    ("partitioned", dict(wave_order="partitioned")),
    ("per_opcode_launch", dict(launch_mode="per_opcode")),
    ("separate_topk_finalize_combine", dict(flags=mk.MK_SCHED_SEPARATE_TOPK | mk.MK_SCHED_SEPARATE_FINALIZE
                                            | mk.MK_SCHED_SEPARATE_COMBINE)),
    ("static_attention", dict(flags=mk.MK_SCHED_STATIC_ATTN)),
    ("static_moe", dict(flags=mk.MK_SCHED_STATIC_MOE)),
    ("shared_attention", dict(flags=mk.MK_SCHED_SHARED_ATTN)),
]
_SCHED_WL = W.Workload("moe30b-shape-sched", MOE_SMALL, batch=2, ctx="list:100,77", steps=2, seed=16)
_sched_state = {}


@pytest.mark.parametrize("name,kw", SCHEDULES, ids=[s[0] for s in SCHEDULES])
def test_schedule_variant_matches_oracle(name, kw):
    wl = _SCHED_WL
    if "oracle" not in _sched_state:
        _sched_state["oracle"] = O.Weights(wl, cache_limit=4 << 30)
    eng = _engine(wl, opts=mk.make_opts(**kw))
    first = eng.decode(inputs=eng.step_inputs()).clone()
    assert eng.status().code == 0
    if name == "tuned":
        _sched_state["tuned"] = first
    elif "tuned" in _sched_state:
        assert torch.equal(first, _sched_state["tuned"]), name
    eng.close()
    eng = _engine(wl, opts=mk.make_opts(**kw))
    run_teacher_forced(eng, 2, W_oracle=_sched_state["oracle"]).check()


def test_moe30b_shape_bs8_long_ragged_contexts():
    """8 sequences of up to 16,380 cached keys: the block table (B x max_blocks
    > 2048 entries) is read from memory rather than LDS, and the attention
    splits sit at their LDS cap (960 keys)."""
    wl = W.Workload("moe30b-shape-bs8-16k", MOE_SMALL, batch=8,
                    ctx="list:16380,9000,12001,700,15000,4000,16100,2048", steps=2, seed=21)
    eng = _engine(wl)
    assert wl.batch * eng.max_blocks > 2048
    tasks, _ = mk.mk_plan_schedule(eng.mkcfg, 8, eng.max_blocks, mk.make_opts(flags=mk.MK_SCHED_STATIC_ATTN), 256)
    ns = max(t.split for t in tasks if t.op == mk.OPCODES.index("ATTN_DECODE")) + 1
    assert -(-eng.max_blocks * 16 // ns) > 900, ns        # splits of about 960 keys
    run_teacher_forced(eng, 2, W_oracle=O.Weights(wl, cache_limit=8 << 30)).check()


def test_moe30b_shape_bs8_concentrated_routing():
    """A router bias with Zipf ranks concentrates the routing (about 21
    distinct experts per layer at bs=8 instead of about 51), as in real
    traffic; parity holds with the bias in the logits."""
    from dataclasses import replace
    wl = W.Workload("moe30b-shape-bs8-zipf", replace(MOE_SMALL, name="moe30b-shape-zipf", router_zipf=1.2),
                    batch=8, ctx="loguniform:100:900", steps=2, seed=23)
    eng = _engine(wl)
    rep = run_teacher_forced(eng, 2, W_oracle=O.Weights(wl, cache_limit=4 << 30))
    rep.check()
    ids = eng.tap("topk_ids").cpu().numpy()[:2 * 8 * 8].reshape(2, 8 * 8)
    distinct = [len(set(ids[l].tolist())) for l in range(2)]
    assert max(distinct) < 40, distinct


SWA_4L = W.ModelConfig(name="moe30b-swa4096-4l", n_layers=4, d_model=2048, n_q_heads=32, n_kv_heads=4,
                       head_dim=128, vocab=2048, n_experts=128, top_k=8, expert_inter=768,
                       swa_window=4096, swa_period=4)


def test_sliding_window_4096_at_262k_context():
    """Layers 0-2 see the 4096 most recent keys, layer 3 all 262,145: RoPE at
    positions past 262K, hundreds of 960-key splits per KV group feeding the
    combine, and the block table read from memory."""
    wl = W.Workload("moe30b-swa-262k", SWA_4L, batch=1, ctx="fixed:262144", steps=2, seed=22)
    eng = _engine(wl)
    assert eng.max_blocks > 2048
    rep = run_teacher_forced(eng, 2, W_oracle=O.Weights(wl, cache_limit=4 << 30))
    rep.check()
    assert rep.compared == 2


def test_dense1b_full_16_layers_tied_vocab():
    """The dense Llama-1B-shaped decoder at its real size: 16 sequential
    pre-norm layers, head dim 64, the tied 128,256-row LM head, 4K context."""
    wl = W.WORKLOADS["dense1b"]
    eng = _engine(wl, steps=2)
    rep = run_teacher_forced(eng, 2, W_oracle=O.Weights(wl, cache_limit=16 << 30))
    rep.check()
    assert rep.compared == 2


def test_watchdog_reports_timeout_and_recovers():
    wl = W.WORKLOADS["tiny"]
    eng = _engine(wl)
    inp = eng.step_inputs()
    ref = eng.decode(inputs=inp).clone()
    assert eng.status().code == 0
    mk.mk_build_schedule(eng.h, 1, mk.make_opts(timeout_ms=50, flags=mk.MK_SCHED_UNREACHABLE_WAIT))
    eng.decode(inputs=inp)
    st = eng.status()
    # the first wait to time out is reported: the blocked task (0) or one of
    # the tasks that wait on its workgroup's later work, whichever polls first
    assert st.code == mk.MK_E_TIMEOUT
    assert 0 <= st.task and st.value < st.target
    assert eng.status().code == 0          # the error record was cleared
    mk.mk_build_schedule(eng.h, 1, mk.make_opts())
    again = eng.decode(inputs=inp).clone()
    assert eng.status().code == 0
    assert torch.equal(ref, again)


def test_bad_page_id_is_reported_not_faulted():
    wl = W.WORKLOADS["tiny"]
    eng = _engine(wl)
    t, pos, sl = eng.step_inputs()
    saved = eng.block_tables.clone()
    eng.block_tables[0, int(pos[0]) // 16] = eng.plan.num_pages + 5
    eng.decode(inputs=(t, pos, sl))
    assert eng.status().code == mk.MK_E_DEVICE
    eng.block_tables.copy_(saved)


def test_full_size_moe30b_first_step():
    """The 48-layer 30B/3.3B-active model at 8K context, step 0, all logits."""
    wl = W.WORKLOADS["moe30b"]
    eng = _engine(wl, steps=4, verbose=True)
    Wo = O.Weights(wl, cache_limit=0)
    seq = O.new_sequence(eng.slot_seq[0].seq_id, eng.slot_seq[0].ctx)
    tok = eng.slot_seq[0].token
    logits = eng.decode([tok])
    assert eng.status().code == 0
    say("oracle: full-size step 0 (lazy weights)")
    res = O.decode_one(wl, Wo, seq, tok, keep_cache=False)
    rep = Report()
    compare_step(eng, [res], logits, rep, [0])
    say(f"full-size: logit err/std {rep.worst_logit_ratio:.2e} router {rep.worst_router_err:.1e} "
        f"taps {rep.worst_tap_ratio:.1e} argmax {rep.argmax_equal}/{rep.compared} flips {rep.exempt_flips}")
    if rep.exempt_flips:
        pytest.skip("an exempt near-tie routing flip; logits not comparable this step")
    rep.check()
