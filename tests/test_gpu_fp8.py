"""FP8 expert weights on the GPU: the stored codes and scales, and parity of
the decode path with the oracle, which decodes every E4M3 code from the
format's definition and multiplies by its row scale in float64."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import decode as O
from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W
from tests.parity import Report, compare_step, run_teacher_forced, say

pytestmark = pytest.mark.gpu

# the 30B model's expert geometry (d 2048, 128 experts of 768), two layers
MOE_SMALL_FP8 = W.ModelConfig(name="moe30b-shape-2l-fp8", n_layers=2, d_model=2048, n_q_heads=32, n_kv_heads=4,
                              head_dim=128, vocab=4096, n_experts=128, top_k=8, expert_inter=768,
                              expert_fp8=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu_available):
    mk.load()
    yield


def _engine(wl, **kw):
    from persistent_moe_amd.runner import DecodeEngine
    say("engine", wl.name, "B", wl.batch, kw)
    return DecodeEngine(wl, **kw)


def test_stored_codes_and_scales_equal_the_cpu_quantization():
    wl = W.Workload("moe30b-shape-fp8-ctx40", MOE_SMALL_FP8, batch=1, ctx="fixed:40", steps=1, seed=31)
    eng = _engine(wl)
    shapes = W.weight_shapes(wl.model)
    for l in range(wl.model.n_layers):
        for name in ("w_upgate", "w_down"):
            assert eng.layers[l][name].dtype == torch.uint8
            for e in (0, 77, 127):
                w = torch.empty(shapes[name], dtype=torch.bfloat16)
                mean, std = W.tensor_dist(name)
                W.fill_normal_(w, W.tensor_key(wl.seed, name, l, e), mean, std)
                codes, scale = W.quantize_e4m3_rows(w)
                assert torch.equal(eng.layers[l][name][e].cpu(), codes), (l, name, e)
                assert torch.equal(eng.layers[l][name + "_scale"][e].cpu(), scale), (l, name, e)
    eng.close()


def test_tiny_moe_fp8_experts_all_steps():
    """d 256 and expert width 128: both GEMVs read one partial 1024-element chunk."""
    wl = W.WORKLOADS["tiny"].with_(name="tiny-moe-fp8", model=replace(W.TINY_MOE, expert_fp8=True))
    eng = _engine(wl)
    rep = run_teacher_forced(eng, wl.steps)
    rep.check()
    assert rep.compared == wl.steps


def test_moe30b_shape_fp8_experts_ragged_context():
    """Gate/up rows of 2048 codes (two chunks), down rows of 768 (one partial chunk)."""
    wl = W.Workload("moe30b-shape-fp8-ctx333", MOE_SMALL_FP8, batch=1, ctx="fixed:333", steps=3, seed=32)
    eng = _engine(wl)
    run_teacher_forced(eng, 3).check()


def test_fp8_experts_with_few_workgroups():
    wl = W.Workload("moe30b-shape-fp8-nw24", MOE_SMALL_FP8, batch=1, ctx="fixed:100", steps=2, seed=33)
    eng = _engine(wl, opts=mk.make_opts(n_workgroups=24))
    run_teacher_forced(eng, 2).check()


def test_tiny_moe_fp8_experts_two_rows():
    """Two batch rows take the MFMA form of the FP8 GEMV (one partial chunk)."""
    wl = W.Workload("tiny-moe-fp8-bs2", replace(W.TINY_MOE, expert_fp8=True), batch=2, ctx="list:64,37",
                    steps=4, seed=34)
    eng = _engine(wl)
    rep = run_teacher_forced(eng, wl.steps)
    rep.check()
    assert rep.rows == 8


def test_moe30b_shape_fp8_experts_bs8_ragged_with_swap():
    wl = W.Workload("moe30b-shape-fp8-bs8", MOE_SMALL_FP8, batch=8, ctx="loguniform:20:700", steps=4, seed=35,
                    swap_every=2)
    eng = _engine(wl)
    rep = run_teacher_forced(eng, 4)
    rep.check()
    assert rep.rows == 32


@pytest.mark.parametrize("ug,dn", [(0, 0), (100, 200)])
def test_fp8_experts_bs8_few_workgroups_and_ragged_items(ug, dn):
    wl = W.Workload(f"moe30b-shape-fp8-bs8-nw40-{ug}", MOE_SMALL_FP8, batch=8, ctx="loguniform:30:500", steps=2,
                    seed=36 + ug)
    eng = _engine(wl, opts=mk.make_opts(n_workgroups=40, moe_ug_pairs=ug, moe_dn_rows=dn))
    run_teacher_forced(eng, 2).check()


def test_full_size_moe30b_fp8_first_step():
    """The 48-layer model with FP8 experts at 8K context, step 0, all logits,
    in the launch configuration the benchmark times."""
    wl = W.WORKLOADS["moe30b_fp8"]
    eng = _engine(wl, steps=4, verbose=True)
    Wo = O.Weights(wl, cache_limit=0)
    seq = O.new_sequence(eng.slot_seq[0].seq_id, eng.slot_seq[0].ctx)
    tok = eng.slot_seq[0].token
    logits = eng.decode([tok])
    assert eng.status().code == 0
    say("oracle: full-size FP8 step 0 (lazy weights)")
    res = O.decode_one(wl, Wo, seq, tok, keep_cache=False)
    rep = Report()
    compare_step(eng, [res], logits, rep, [0])
    say(f"full-size fp8: logit err/std {rep.worst_logit_ratio:.2e} router {rep.worst_router_err:.1e} "
        f"taps {rep.worst_tap_ratio:.1e} argmax {rep.argmax_equal}/{rep.compared} flips {rep.exempt_flips}")
    if rep.exempt_flips:
        pytest.skip("an exempt near-tie routing flip; logits not comparable this step")
    rep.check()
    eng.close()
