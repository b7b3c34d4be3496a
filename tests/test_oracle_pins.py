"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against a closed form, an invariant, a special
case that reduces to a textbook or library routine, or brute force on a tiny
input, so that a dropped term, a wrong sign or index, or a transposed operand
in ``oracle/decode.py`` fails at least one of them.
"""
import itertools
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import decode as O
from persistent_moe_amd import workloads as W

rng = np.random.default_rng(1234)


# ----------------------------------------------------------------- bf16 rounding
def test_bf16_round_matches_torch_conversion():
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    ours = O.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1.
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert O.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert O.bf16_round(np.array([-1.0 - 3 * 2.0 ** -8]))[0] == -1.0 - 2.0 ** -6


# ----------------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    d, c, eps = 64, 0.01, 1e-2
    g = 1.0 + rng.standard_normal(d) * 0.1
    out = O.rms_norm(np.full(d, c), g, eps)
    assert np.allclose(out, g * c / math.sqrt(c * c + eps), rtol=0, atol=1e-15)


def test_rmsnorm_worked_example():
    out = O.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(out, [3 / r, 8 / r], rtol=1e-15)


def test_rmsnorm_scale_invariant_without_eps():
    x = rng.standard_normal(128)
    g = rng.standard_normal(128)
    assert np.allclose(O.rms_norm(7.5 * x, g, 0.0), O.rms_norm(x, g, 0.0), rtol=1e-13)


# -------------------------------------------------------------------------- RoPE
def test_rope_identity_at_position_zero():
    x = rng.standard_normal((3, 16))
    assert np.array_equal(O.rope(x, 0, 1e4), x)


def test_rope_pairs_frequencies_and_direction():
    # hd = 4, theta = 100: pair (0, 2) turns by pos rad, pair (1, 3) by pos/10 rad.
    p = 3
    e0 = O.rope(np.array([[1.0, 0, 0, 0]]), p, 100.0)[0]
    assert np.allclose(e0, [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    e1 = O.rope(np.array([[0, 1.0, 0, 0]]), p, 100.0)[0]
    assert np.allclose(e1, [0, math.cos(p / 10), 0, math.sin(p / 10)], atol=1e-15)
    e2 = O.rope(np.array([[0, 0, 1.0, 0]]), p, 100.0)[0]
    assert np.allclose(e2, [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_preserves_norm_and_depends_on_relative_position():
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    assert np.allclose(np.linalg.norm(O.rope(q, 777, 1e4)), np.linalg.norm(q))
    a = O.rope(q, 50, 1e4)[0] @ O.rope(k, 20, 1e4)[0]
    b = O.rope(q, 1050, 1e4)[0] @ O.rope(k, 1020, 1e4)[0]
    assert abs(a - b) < 1e-9


# --------------------------------------------------------------------- attention
def test_attention_single_key_returns_v():
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((1, 2, 8))
    V = rng.standard_normal((1, 2, 8))
    out = O.attention_decode(q, K, V)
    for i in range(4):
        assert np.allclose(out[i], V[0, i // 2])


def test_attention_identical_keys_give_mean_of_values():
    q = rng.standard_normal((2, 8))
    K = np.repeat(rng.standard_normal((1, 1, 8)), 5, axis=0)
    V = rng.standard_normal((5, 1, 8))
    out = O.attention_decode(q, K, V)
    assert np.allclose(out, np.broadcast_to(V[:, 0].mean(0), (2, 8)))


def test_attention_two_keys_closed_form_scale():
    hd, a = 16, 3.0
    q = np.zeros((1, hd)); q[0, 0] = a
    K = np.zeros((2, 1, hd)); K[0, 0, 0] = 1.0
    V = rng.standard_normal((2, 1, hd))
    p1 = 1.0 / (1.0 + math.exp(-a / math.sqrt(hd)))
    out = O.attention_decode(q, K, V)[0]
    assert np.allclose(out, p1 * V[0, 0] + (1 - p1) * V[1, 0], atol=1e-14)


def test_attention_gqa_head_mapping():
    # Hq = 4, Hkv = 2: query head i reads kv head i // 2.
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((3, 2, 8))
    V = np.zeros((3, 2, 8)); V[:, 0, :] = 1.0; V[:, 1, :] = 2.0
    out = O.attention_decode(q, K, V)
    assert np.allclose(out[:, 0], [1, 1, 2, 2])


def test_attention_dominant_score_selects_its_value():
    q = np.zeros((1, 4)); q[0, 1] = 1.0
    K = np.zeros((3, 1, 4)); K[2, 0, 1] = 400.0
    V = rng.standard_normal((3, 1, 4))
    assert np.allclose(O.attention_decode(q, K, V)[0], V[2, 0], atol=1e-12)


@pytest.mark.parametrize("cuts", [[0, 7, 16, 33], [0, 1, 2, 33], [0, 33]])
def test_split_combine_equals_monolithic(cuts):
    q = rng.standard_normal((8, 32)) * 2
    K = rng.standard_normal((33, 2, 32))
    V = rng.standard_normal((33, 2, 32))
    parts = [O.attention_split(q, K[a:b], V[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.allclose(O.attention_combine(parts), O.attention_decode(q, K, V), atol=1e-13)


# ------------------------------------------------------------------ router/top-k
def test_route_weights_and_probs_sum_to_one():
    for _ in range(20):
        r = O.route(rng.standard_normal(128), 8)
        assert abs(r.weights.sum() - 1) < 1e-14 and abs(r.probs.sum() - 1) < 1e-14


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (5, 1)])
def test_route_brute_force_over_all_subsets(E, k):
    for _ in range(30):
        logits = rng.standard_normal(E)
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(logits[list(s)]))
        r = O.route(logits, k)
        assert set(r.ids.tolist()) == set(best)
        ex = np.exp(logits[list(r.ids)])
        assert np.allclose(r.weights, ex / ex.sum(), rtol=1e-13)
        srt = np.sort(logits)[::-1]
        assert math.isclose(r.margin, srt[k - 1] - srt[k], rel_tol=1e-12)


def test_route_ties_go_to_lower_expert_id():
    r = O.route(np.array([0.5, 1.0, 1.0, 1.0, 0.1]), 2)
    assert r.ids.tolist() == [1, 2] and r.margin == 0.0


def test_route_k_equals_E_is_full_softmax_gating():
    logits = rng.standard_normal(6)
    r = O.route(logits, 6)
    assert np.allclose(r.weights[np.argsort(r.ids)], r.probs, rtol=1e-14)


# ------------------------------------------------------------------ SwiGLU / MoE
def test_swiglu_worked_example_gate_then_up():
    h = np.array([1.0, 2.0])
    w_ug = np.array([[1.0, 0.0],    # gate row -> g = 1
                     [0.0, 1.0]])   # up row   -> u = 2
    w_d = np.array([[1.0], [2.0]])
    act = 2.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(O.swiglu(h, w_ug, w_d), [act, 2 * act], rtol=1e-15)


def test_projection_of_small_integers_is_exact():
    A = rng.integers(-8, 8, (64, 96)).astype(np.float64)
    x = rng.integers(-8, 8, 96).astype(np.float64)
    ref = [sum(int(A[i, j]) * int(x[j]) for j in range(96)) for i in range(64)]
    assert np.array_equal(A @ x, np.array(ref, dtype=np.float64))


def test_moe_identical_experts_reduce_to_dense_swiglu():
    d, I, E = 16, 8, 4
    h = rng.standard_normal(d)
    ug = rng.standard_normal((2 * I, d)) * 0.3
    dn = rng.standard_normal((d, I)) * 0.3
    r = O.route(rng.standard_normal(E), E)
    out = O.moe(h, r, lambda e: (ug, dn))
    assert np.allclose(out, O.swiglu(h, ug, dn), atol=1e-14)


def test_moe_top1_is_the_selected_expert():
    d, I, E = 16, 8, 5
    h = rng.standard_normal(d)
    experts = [(rng.standard_normal((2 * I, d)), rng.standard_normal((d, I))) for _ in range(E)]
    logits = rng.standard_normal(E)
    out = O.moe(h, O.route(logits, 1), lambda e: experts[e])
    e = int(np.argmax(logits))
    assert np.allclose(out, O.swiglu(h, *experts[e]))


def test_moe_two_experts_weighted_by_renormalised_softmax():
    d, I = 8, 4
    h = rng.standard_normal(d)
    experts = [(rng.standard_normal((2 * I, d)), rng.standard_normal((d, I))) for _ in range(3)]
    logits = np.array([0.3, 1.2, 0.9])
    out = O.moe(h, O.route(logits, 2), lambda e: experts[e])
    w1 = 1.0 / (1.0 + math.exp(0.9 - 1.2))
    ref = w1 * O.swiglu(h, *experts[1]) + (1 - w1) * O.swiglu(h, *experts[2])
    assert np.allclose(out, ref, atol=1e-13)


# ---------------------------------------------------------- whole-step structure
class _HandWeights(O.Weights):
    """Hand-built weights for structural pins (shapes of a tiny model)."""

    def __init__(self, wl, tensors):
        super().__init__(wl)
        self.t = tensors

    def layer(self, name, layer):
        return self.t[name][layer]

    def expert(self, layer, e):
        return self.t["experts"][layer][e]

    def dense_ffn(self, layer):
        return self.t["w_upgate"][layer], self.t["w_down"][layer]

    def final_norm(self):
        return self.t["final_norm"]

    def embed_row(self, token):
        return self.t["embed"][token]

    def lm_head_rows(self, r0, r1):
        return self.t["lm_head"][r0:r1]


def _tiny_wl(**kw):
    cfg = W.ModelConfig(name="pin", n_layers=2, d_model=8, n_q_heads=2, n_kv_heads=1,
                        head_dim=4, vocab=5, n_experts=3, top_k=2, expert_inter=4, **kw)
    return W.Workload("pin", cfg, batch=1, ctx="fixed:3", steps=2, seed=7)


def _hand_tensors(cfg, zero_branches=False):
    L, d, V = cfg.n_layers, cfg.d_model, cfg.vocab
    s = 0.0 if zero_branches else 0.3
    t = {
        "attn_norm": [1 + 0.1 * rng.standard_normal(d) for _ in range(L)],
        "ffn_norm": [1 + 0.1 * rng.standard_normal(d) for _ in range(L)],
        "w_qkv": [rng.standard_normal((cfg.qkv_rows, d)) * 0.3 for _ in range(L)],
        "w_o": [rng.standard_normal((d, cfg.attn_dim)) * s for _ in range(L)],
        "w_router": [rng.standard_normal((cfg.n_experts, d)) for _ in range(L)],
        "experts": [[(rng.standard_normal((2 * cfg.expert_inter, d)) * s,
                      rng.standard_normal((d, cfg.expert_inter)) * 0.3)
                     for _ in range(cfg.n_experts)] for _ in range(L)],
        "final_norm": 1 + 0.1 * rng.standard_normal(d),
        "embed": rng.standard_normal((V, d)),
        "lm_head": rng.standard_normal((V, d)),
    }
    return t


def test_step_with_silent_branches_is_norm_then_lm_head():
    wl = _tiny_wl()
    t = _hand_tensors(wl.model, zero_branches=True)
    Wt = _HandWeights(wl, t)
    seq = O.new_sequence(0, 3)
    res = O.decode_one(wl, Wt, seq, token=4)
    x = t["embed"][4]
    ref = t["lm_head"] @ (x / math.sqrt(np.mean(x * x) + wl.model.rms_eps) * t["final_norm"])
    assert np.allclose(res.logits, ref, atol=1e-13)
    assert res.token == int(np.argmax(ref)) and seq.length == 4


def test_step_parallel_residual_sums_both_branches():
    wl = _tiny_wl()
    t = _hand_tensors(wl.model)
    Wt = _HandWeights(wl, t)
    res = O.decode_one(wl, Wt, O.new_sequence(0, 3), token=1)
    x = t["embed"][1]
    for l, tap in enumerate(res.layers):
        assert np.allclose(tap.x_out, x + tap.attn_out + tap.ffn_out, atol=1e-14)
        # both branches read the same normed input
        assert np.allclose(tap.h, O.rms_norm(x, t["attn_norm"][l], wl.model.rms_eps))
        x = tap.x_out


def test_step_appends_rotated_bf16_key_and_attends_to_it():
    wl = _tiny_wl()
    cfg = wl.model
    t = _hand_tensors(cfg)
    # zero query rows: every visible key gets the same score, so attention is
    # the mean of all visible values, the new one included.
    for l in range(cfg.n_layers):
        t["w_qkv"][l][:cfg.n_q_heads * cfg.head_dim] = 0.0
    Wt = _HandWeights(wl, t)
    seq = O.new_sequence(0, 3)
    res = O.decode_one(wl, Wt, seq, token=2)
    for l, tap in enumerate(res.layers):
        qkv = t["w_qkv"][l] @ tap.h
        k = qkv[cfg.n_q_heads * cfg.head_dim:(cfg.n_q_heads + 1) * cfg.head_dim].reshape(1, -1)
        assert np.array_equal(seq.appended_k[l][0], O.bf16_round(O.rope(k, 3, cfg.rope_theta)))
        K, V = O.cached_kv(wl, seq, l, 0, 4)
        assert K.shape[0] == 4
        assert np.allclose(tap.attn.reshape(cfg.n_q_heads, -1), V[:, 0].mean(0), atol=1e-14)


def test_sliding_window_boundary():
    # window 1: only the token itself is visible, so attention returns its value.
    wl = _tiny_wl(swa_window=1, swa_period=4)
    cfg = wl.model
    t = _hand_tensors(cfg)
    res = O.decode_one(wl, _HandWeights(wl, t), O.new_sequence(0, 3), token=0)
    for l in (0, 1):       # layers 0..2 of a period of 4 are windowed
        assert np.allclose(res.layers[l].attn.reshape(cfg.n_q_heads, -1), res.layers[l].v_new[0])
    # a window at least the context length equals global attention
    wl_big = _tiny_wl(swa_window=64, swa_period=4)
    r_big = O.decode_one(wl_big, _HandWeights(wl_big, t), O.new_sequence(0, 3), token=0)
    r_glob = O.decode_one(_tiny_wl(), _HandWeights(_tiny_wl(), t), O.new_sequence(0, 3), token=0)
    assert np.allclose(r_big.logits, r_glob.logits, atol=1e-13)


def test_sequential_block_applies_second_norm_to_updated_residual():
    wl = _tiny_wl()
    cfg = W.ModelConfig(name="pin-seq", n_layers=1, d_model=8, n_q_heads=2, n_kv_heads=1,
                        head_dim=4, vocab=5, ffn_inter=4, parallel_block=False)
    wl = W.Workload("pin-seq", cfg, batch=1, ctx="fixed:2", steps=1, seed=7)
    t = _hand_tensors(_tiny_wl().model)
    t["w_qkv"] = [rng.standard_normal((cfg.qkv_rows, 8)) * 0.3]
    t["w_o"] = [rng.standard_normal((8, cfg.attn_dim)) * 0.3]
    t["w_upgate"] = [rng.standard_normal((8, 8)) * 0.3]
    t["w_down"] = [rng.standard_normal((8, 4)) * 0.3]
    res = O.decode_one(wl, _HandWeights(wl, t), O.new_sequence(0, 2), token=3)
    tap = res.layers[0]
    x1 = t["embed"][3] + tap.attn_out
    h2 = O.rms_norm(x1, t["ffn_norm"][0], cfg.rms_eps)
    assert np.allclose(tap.ffn_out, O.swiglu(h2, t["w_upgate"][0], t["w_down"][0]), atol=1e-14)
    assert np.allclose(tap.x_out, x1 + tap.ffn_out, atol=1e-14)


# ------------------------------------------------------------------ whole decode
def test_tiny_greedy_decode_repeatable_from_seed():
    wl = W.WORKLOADS["tiny"]
    fed1, res1 = O.greedy_decode(wl, 4)
    fed2, res2 = O.greedy_decode(wl, 4)
    assert fed1 == fed2
    for a, b in zip(res1, res2):
        assert np.array_equal(a[0].logits, b[0].logits)


def test_batch_rows_equal_single_sequence_runs():
    wl = W.WORKLOADS["tiny"].with_(batch=3, ctx="loguniform:20:90")
    Wt = O.Weights(wl)
    plan = W.plan_batch(wl, 2)
    seqs = [O.new_sequence(plan.slots[b][0][1].seq_id, plan.slots[b][0][1].ctx) for b in range(3)]
    toks = [plan.slots[b][0][1].token for b in range(3)]
    res = O.decode_step(wl, Wt, seqs, toks)
    for b in range(3):
        s1 = O.new_sequence(plan.slots[b][0][1].seq_id, plan.slots[b][0][1].ctx)
        r1 = O.decode_one(wl, Wt, s1, toks[b])
        assert np.array_equal(r1.logits, res[b].logits)


# ------------------------------------------------------ cache and tied LM head
# The oracle reads the pre-filled cache through ``cached_kv`` (a row offset
# into the KV stream of the sequence and layer) and the tied LM head through
# the embedding stream.  Both are pinned to whole-tensor draws of the
# generator, sliced with numpy, so an offset, layer or stream mix-up fails.
def _kv_rows(wl, seq_id, layer, which, ctx):
    return W.gen_kv(wl.seed, wl.model, seq_id, layer, which, 0, ctx).float().numpy().astype(np.float64)


@pytest.mark.parametrize("p0,p1", [(0, 40), (13, 29), (39, 40), (0, 1), (17, 18)])
def test_cached_kv_prefill_rows_equal_generator_rows(p0, p1):
    wl = W.WORKLOADS["tiny"]
    seq = O.new_sequence(3, 40)
    for layer in (0, 1):
        K, V = O.cached_kv(wl, seq, layer, p0, p1, keep=False)
        assert np.array_equal(K, _kv_rows(wl, 3, layer, "k", 40)[p0:p1])
        assert np.array_equal(V, _kv_rows(wl, 3, layer, "v", 40)[p0:p1])
    # another layer, sequence or operand is another stream
    K1, _ = O.cached_kv(wl, seq, 1, 0, 40, keep=False)
    K0, V0 = O.cached_kv(wl, seq, 0, 0, 40, keep=False)
    assert not np.array_equal(K0, K1) and not np.array_equal(K0, V0)
    assert not np.array_equal(K0, O.cached_kv(wl, O.new_sequence(4, 40), 0, 0, 40, keep=False)[0])


def test_cached_kv_straddles_prefill_and_appended_entries():
    wl = W.WORKLOADS["tiny"]
    cfg = wl.model
    seq = O.new_sequence(5, 40)
    app_k = [np.full((cfg.n_kv_heads, cfg.head_dim), 100.0 + i) for i in range(3)]
    app_v = [np.full((cfg.n_kv_heads, cfg.head_dim), -100.0 - i) for i in range(3)]
    seq.appended_k[1] = list(app_k)
    seq.appended_v[1] = list(app_v)
    seq.length = 43
    gk, gv = _kv_rows(wl, 5, 1, "k", 40), _kv_rows(wl, 5, 1, "v", 40)
    K, V = O.cached_kv(wl, seq, 1, 35, 43, keep=False)
    assert np.array_equal(K, np.concatenate([gk[35:40], np.stack(app_k)]))
    assert np.array_equal(V, np.concatenate([gv[35:40], np.stack(app_v)]))
    K, V = O.cached_kv(wl, seq, 1, 41, 43, keep=False)
    assert np.array_equal(K, np.stack(app_k[1:])) and np.array_equal(V, np.stack(app_v[1:]))
    # the kept slice of one layer is not served to another range
    K, _ = O.cached_kv(wl, seq, 1, 0, 10)
    K2, _ = O.cached_kv(wl, seq, 1, 10, 20)
    assert np.array_equal(K2, gk[10:20])


def test_tied_lm_head_rows_are_embedding_rows():
    cfg = W.ModelConfig(name="pin-tied", n_layers=1, d_model=64, n_q_heads=2, n_kv_heads=1, head_dim=64,
                        vocab=300, ffn_inter=64, tied_embeddings=True, parallel_block=False)
    wl = W.Workload("pin-tied", cfg, batch=1, ctx="fixed:4", steps=1, seed=9)
    Wt = O.Weights(wl)
    emb = W.gen_tensor(wl.seed, "embed", (cfg.vocab, cfg.d_model)).float().numpy().astype(np.float64)
    for r0, r1 in ((0, 300), (17, 18), (250, 300)):
        assert np.array_equal(Wt.lm_head_rows(r0, r1), emb[r0:r1])
    assert np.array_equal(Wt.embed_row(123), emb[123])
    # untied: the LM head is its own stream
    wu = O.Weights(wl.with_(model=replace(cfg, tied_embeddings=False)))
    assert not np.array_equal(wu.lm_head_rows(0, 300), emb)


# ----------------------------------------------------------------- sampling
def test_greedy_sampling_is_argmax_with_ties_to_lowest_id():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    assert O.sample_token(z, 0.0) == (1, 0.0)
    tok, gap = O.sample_token(np.array([0.1, 0.7, 0.3]), 0.0)
    assert tok == 1 and abs(gap - 0.4) < 1e-15


def test_sampling_uniforms_reference_values():
    # with seed, position and slot 0 the key is fmix32(0) = 0, so u_v is
    # (fmix32(v) / 2^8 + 1/2) / 2^24; MurmurHash3's fmix32(1) is 0x514E28B7
    u = O.sampling_uniforms(0, 0, 0, 2)
    assert u[0] == 0.5 / 2 ** 24 and u[1] == (0x514E28 + 0.5) / 2 ** 24
    a, b = O.sampling_uniforms(7, 100, 3, 1000), O.sampling_uniforms(7, 101, 3, 1000)
    assert np.all((a > 0) & (a < 1)) and not np.array_equal(a, b)
    assert not np.array_equal(a, O.sampling_uniforms(7, 100, 2, 1000))
    assert abs(a.mean() - 0.5) < 0.03


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_temperature_sampling_draws_from_tempered_softmax(T):
    # the Gumbel-max draw over many positions has the frequencies of
    # softmax(logits / T): a chi-square test at 6 dof (p = 1e-4 cut)
    z = np.array([1.0, 0.2, -0.5, 0.9, 0.0, -2.0, 0.4])
    n = 20000
    counts = np.bincount([O.sample_token(z, T, seed=11, position=p)[0] for p in range(n)], minlength=7)
    p = np.exp(z / T) / np.exp(z / T).sum()
    chi2 = float(np.sum((counts - n * p) ** 2 / (n * p)))
    assert chi2 < 27.9, (counts, n * p)


# ------------------------------------------------------------- router bias
def test_router_bias_values_are_zipf_ranks():
    cfg = W.MOE_30B_ZIPF
    b = W.router_bias(5, cfg, 3).float().numpy().astype(np.float64)
    want = np.sort(O.bf16_round(-cfg.router_zipf * np.log(np.arange(cfg.n_experts) + 1.0)))
    assert np.array_equal(np.sort(b), want)            # one expert per rank
    assert not np.array_equal(b, W.router_bias(5, cfg, 4).float().numpy())
    assert W.router_bias(5, W.MOE_30B, 3) is None


def test_router_bias_moves_selection_and_gate_weights():
    # zero router weights: the logits are the bias alone, so the selected
    # experts and their gates are the top-k of the bias
    wl = _tiny_wl()
    t = _hand_tensors(wl.model)
    for l in range(wl.model.n_layers):
        t["w_router"][l] = np.zeros_like(t["w_router"][l])
    bias = np.array([0.1, 1.5, 0.7])

    class Biased(_HandWeights):
        def router_bias(self, layer):
            return bias

    res = O.decode_one(wl, Biased(wl, t), O.new_sequence(0, 3), token=2)
    for tap in res.layers:
        assert tap.route.ids.tolist() == [1, 2]
        w1 = 1.0 / (1.0 + math.exp(0.7 - 1.5))
        assert np.allclose(tap.route.weights, [w1, 1 - w1], atol=1e-14)
        assert np.allclose(tap.router_logits, bias)


# ---------------------------------------------------------------- FP8 experts
def test_e4m3_decode_matches_the_library_conversion_on_every_code():
    codes = np.arange(256)
    ours = O.e4m3_decode(codes)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)].astype(np.float64))


def test_e4m3_decode_closed_form_values():
    v = O.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0xB8, 0x7F]))
    assert v[0] == 0.0 and v[1] == 2.0 ** -9 and v[2] == 7 * 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 1.0 and v[5] == 1.5 and v[6] == 448.0 and v[7] == -1.0 and np.isnan(v[8])


def test_e4m3_quantizer_rounds_like_a_correct_float8_conversion():
    """With a row maximum of 448 the scale is 1 and the codes must be the
    round-to-nearest-even E4M3 conversion of each float32 weight, which
    torch's CPU conversion computes in software: checked on log-spaced
    magnitudes, exact ties (normal and subnormal), zeros and the maximum."""
    rng = np.random.default_rng(5)
    mags = np.exp2(rng.uniform(-13, np.log2(448.0), 4000))
    grid = O.e4m3_decode(np.arange(0x7F))                        # the non-negative finite values, ascending
    ties = (grid[:-1] + grid[1:]) / 2                             # every midpoint of the grid
    v = np.concatenate([mags, ties, grid, [0.0, 448.0]]).astype(np.float32)
    v = np.where(rng.random(v.size) < 0.5, -v, v).astype(np.float32)
    v = np.concatenate([v, np.float32([-0.0, 448.0])])
    w = torch.from_numpy(v.reshape(1, -1))
    codes, scale = W.quantize_e4m3_rows(w)
    assert scale.item() == 1.0
    ref = w.to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(codes, ref)
    # with any row maximum, that element maps to the largest code, +-448
    rows = torch.from_numpy(rng.standard_normal((64, 300)).astype(np.float32) * np.exp2(rng.uniform(-20, 20, (64, 1))))
    codes, scale = W.quantize_e4m3_rows(rows)
    assert torch.equal((codes & 0x7F).amax(dim=1), torch.full((64,), 0x7E, dtype=torch.uint8))


def test_fp8_expert_rows_round_trip_within_half_a_code_step():
    wl = W.WORKLOADS["tiny"].with_(model=replace(W.TINY_MOE, expert_fp8=True))
    ug_q, dn_q = O.Weights(wl).expert(1, 3)
    ug = W.gen_tensor(wl.seed, "w_upgate", W.weight_shapes(wl.model)["w_upgate"], layer=1, expert=3).double().numpy()
    # each row's largest magnitude maps to 448 and is exact; every element is
    # within half an E4M3 step (2**-4 relative for normal values) of its weight
    amax = np.abs(ug).max(axis=1, keepdims=True)
    assert np.allclose(np.abs(ug_q).max(axis=1, keepdims=True), amax, rtol=1e-6)
    assert np.all(np.abs(ug_q - ug) <= np.maximum(np.abs(ug) * 2.0 ** -4, amax / 448 * 2.0 ** -9) + 1e-12)
    assert not np.array_equal(ug_q, ug)
    assert dn_q.shape == W.weight_shapes(wl.model)["w_down"]
