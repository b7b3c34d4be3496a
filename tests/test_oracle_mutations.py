"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in test_oracle_pins.py catch each one.  Nothing here touches the GPU path."""
import json
import math
import os

import numpy as np
import pytest

from oracle import decode as O
from persistent_moe_amd import workloads as W
from tests import test_oracle_pins as P

_orig = {n: getattr(O, n) for n in ("rms_norm", "rope", "attention_decode", "route", "swiglu",
                                    "moe", "bf16_round", "attention_combine")}


def _rms_sum(x, g, eps):
    return x / np.sqrt(np.sum(x * x) + eps) * g


def _rms_eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x)) + eps) * g


def _rope_adjacent(x, pos, theta):
    hd = x.shape[-1]
    i = np.arange(hd // 2, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / hd)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_sign(x, pos, theta):
    return _orig["rope"](x, -pos, theta)


def _rope_freq(x, pos, theta):
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * theta ** (-1.0 * i / hd)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * np.cos(ang) - b * np.sin(ang), b * np.cos(ang) + a * np.sin(ang)], -1)


def _attn_scale(q, K, V):
    return _orig["attention_decode"](q * math.sqrt(q.shape[1]) / q.shape[1], K, V)


def _attn_mapping(q, K, V):
    Hq, hd = q.shape
    out = np.empty((Hq, hd))
    for i in range(Hq):
        g = i % K.shape[1]
        p = O.softmax(K[:, g, :] @ q[i] / math.sqrt(hd))
        out[i] = p @ V[:, g, :]
    return out


def _route_ties_high(logits, k):
    E = logits.shape[0]
    order = sorted(range(E), key=lambda e: (-logits[e], -e))
    r = _orig["route"](logits, k)
    r.ids = np.array(order[:k])
    r.weights = r.probs[r.ids] / r.probs[r.ids].sum()
    return r


def _route_no_renorm(logits, k):
    r = _orig["route"](logits, k)
    r.weights = r.probs[r.ids]
    return r


def _swiglu_swapped(h, w_ug, w_d):
    inter = w_ug.shape[0] // 2
    return w_d @ (O.silu(w_ug[inter:] @ h) * (w_ug[:inter] @ h))


def _moe_unweighted(h, r, expert):
    return sum(O.swiglu(h, *expert(int(e))) for e in r.ids)


def _bf16_truncate(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.trunc(m * 256.0) / 256.0, e)


def _combine_no_rescale(parts):
    num = sum(p[2] for p in parts)
    den = sum(p[1] for p in parts)
    return num / den[:, None]


MUTATIONS = [
    ("rms_norm", _rms_sum, [P.test_rmsnorm_constant_vector_closed_form]),
    ("rms_norm", _rms_eps_outside, [P.test_rmsnorm_constant_vector_closed_form]),
    ("rope", _rope_adjacent, [P.test_rope_pairs_frequencies_and_direction]),
    ("rope", _rope_sign, [P.test_rope_pairs_frequencies_and_direction]),
    ("rope", _rope_freq, [P.test_rope_pairs_frequencies_and_direction]),
    ("attention_decode", _attn_scale, [P.test_attention_two_keys_closed_form_scale]),
    ("attention_decode", _attn_mapping, [P.test_attention_gqa_head_mapping]),
    ("route", _route_ties_high, [P.test_route_ties_go_to_lower_expert_id]),
    ("route", _route_no_renorm, [P.test_route_weights_and_probs_sum_to_one]),
    ("swiglu", _swiglu_swapped, [P.test_swiglu_worked_example_gate_then_up]),
    ("moe", _moe_unweighted, [P.test_moe_two_experts_weighted_by_renormalised_softmax]),
    ("bf16_round", _bf16_truncate, [P.test_bf16_round_matches_torch_conversion]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, fn, pins):
    monkeypatch.setattr(O, name, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the mutation {fn.__name__} of {name}"


def test_split_combine_pin_catches_missing_rescale(monkeypatch):
    monkeypatch.setattr(O, "attention_combine", _combine_no_rescale)
    with pytest.raises(AssertionError):
        P.test_split_combine_equals_monolithic([0, 7, 16, 33])


def test_window_off_by_one_is_caught(monkeypatch):
    orig = W.ModelConfig.layer_window
    monkeypatch.setattr(W.ModelConfig, "layer_window", lambda self, l: orig(self, l) + 1 if orig(self, l) else 0)
    with pytest.raises(AssertionError):
        P.test_sliding_window_boundary()


def test_oracle_reproduces_golden_greedy_decode():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_greedy.json")
    gold = json.load(open(path))
    fed, res = O.greedy_decode(W.WORKLOADS["tiny"], 4)
    for g, f, r in zip(gold["steps"], fed, res):
        assert g["fed_token"] == f[0] and g["argmax"] == r[0].token
        assert g["experts"] == [t.route.ids.tolist() for t in r[0].layers]
        assert np.allclose(g["logits_head"], r[0].logits[:8], rtol=0, atol=1e-12)


def _cached_kv_mutant(shift_prefill=0, layer_fixed=None, shift_appended=0):
    """cached_kv with a planted offset, layer or appended-index mistake."""
    def fn(wl, seq, layer, p0, p1, keep=True):
        cfg = wl.model
        parts_k, parts_v = [], []
        if p0 < seq.ctx0:
            q1 = min(p1, seq.ctx0)
            ly = layer if layer_fixed is None else layer_fixed
            parts_k.append(O._f64(W.gen_kv(wl.seed, cfg, seq.seq_id, ly, "k", p0 + shift_prefill, q1 + shift_prefill)))
            parts_v.append(O._f64(W.gen_kv(wl.seed, cfg, seq.seq_id, ly, "v", p0 + shift_prefill, q1 + shift_prefill)))
        if p1 > seq.ctx0:
            a0 = max(p0, seq.ctx0) - seq.ctx0 + shift_appended
            a1 = p1 - seq.ctx0 + shift_appended
            parts_k.append(np.stack(seq.appended_k[layer][a0:a1]))
            parts_v.append(np.stack(seq.appended_v[layer][a0:a1]))
        return np.concatenate(parts_k), np.concatenate(parts_v)
    return fn


@pytest.mark.parametrize("kw", [{"shift_prefill": 1}, {"shift_prefill": -1}, {"layer_fixed": 0},
                                {"shift_appended": 1}, {"shift_appended": -1}],
                         ids=["prefill+1", "prefill-1", "layer0", "appended+1", "appended-1"])
def test_cache_pins_catch_offset_mistakes(monkeypatch, kw):
    monkeypatch.setattr(O, "cached_kv", _cached_kv_mutant(**kw))
    caught = 0
    for pin in (lambda: P.test_cached_kv_prefill_rows_equal_generator_rows(13, 29),
                lambda: P.test_cached_kv_prefill_rows_equal_generator_rows(1, 40),
                P.test_cached_kv_straddles_prefill_and_appended_entries):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the cache mutation {kw}"


def test_tied_head_pin_catches_untied_stream(monkeypatch):
    def rows(self, r0, r1):
        return O._f64(W.gen_tensor(self.seed, "lm_head", (self.cfg.vocab, self.cfg.d_model), rows=slice(r0, r1)))
    monkeypatch.setattr(O.Weights, "lm_head_rows", rows)
    with pytest.raises(AssertionError):
        P.test_tied_lm_head_rows_are_embedding_rows()


def _sample_mutant(kind):
    def fn(logits, temperature, seed=0, position=0, slot=0):
        z = np.asarray(logits, dtype=np.float64)
        if temperature > 0:
            u = O.sampling_uniforms(seed, position, slot, z.shape[0])
            g = -np.log(-np.log(u))
            z = {"noise_sign": z / temperature - g, "temp_times": z * temperature + g,
                 "log_noise": z / temperature + np.log(u)}[kind]
        return int(np.argmax(z)), 0.0
    return fn


@pytest.mark.parametrize("kind", ["noise_sign", "temp_times", "log_noise"])
def test_sampling_pin_catches_planted_mistake(monkeypatch, kind):
    monkeypatch.setattr(O, "sample_token", _sample_mutant(kind))
    caught = 0
    for T in (0.5, 2.0):
        try:
            P.test_temperature_sampling_draws_from_tempered_softmax(T)
        except AssertionError:
            caught += 1
    assert caught > 0, kind


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 8), np.ldexp(m / 8.0, -7))
    return np.where(c & 0x80, -mag, mag)


def _e4m3_no_subnormals(codes):
    v = _orig_e4m3(codes)
    e = (np.asarray(codes) >> 3) & 0xF
    return np.where(e == 0, 0.0, v)


_orig_e4m3 = O.e4m3_decode


@pytest.mark.parametrize("fn", [_e4m3_bias8, _e4m3_no_subnormals])
def test_e4m3_pins_catch_planted_mistakes(monkeypatch, fn):
    monkeypatch.setattr(O, "e4m3_decode", fn)
    caught = 0
    for pin in (P.test_e4m3_decode_matches_the_library_conversion_on_every_code,
                P.test_e4m3_decode_closed_form_values):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0
