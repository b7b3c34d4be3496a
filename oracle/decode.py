"""CPU oracle of one decode step of a parallel-block MoE transformer.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The product path (the HIP library and its binding) never
imports, links or calls it.

What it computes is the plain definition of a decode step as the persistent
decode megakernel pages describe the model and its task types (page 1,
"One kernel for the full decode step" and "The calling convention that makes
it hand-writable"; page 4, the list of 16 task types): for every sequence,
embedding lookup, then per layer RMSNorm, QKV projection with rotary position
embedding, append of the new key and value to the cache, grouped-query
attention over the cached keys, output projection, router GEMM, top-k
selection with softmax-renormalised gates, the SwiGLU experts and their
weighted combination, the parallel residual update, and finally a last
RMSNorm and the LM head.  The pages give no formulas; the readings taken where
they are silent are listed in the module constants and function docstrings
(RMSNorm eps, rotate-half RoPE, ties to the lower index, bf16 rounding of the
appended key and value).

Arithmetic is float64 throughout.  Values that are bf16 by definition
(weights, gains, embeddings, the pre-filled cache, and each newly appended key
and value, which are rounded to bf16 when written and read back from the cache)
are held as float64 copies of their bf16 values.  The oracle shares no code
with the GPU path; inputs come from ``persistent_moe_amd.workloads``, which
holds only the seeded generator.

Each sequence is computed on its own, one op after the other, with no
blocking, fusion or reordering; attention is the monolithic softmax over all
visible keys.  ``attention_split`` and ``attention_combine`` restate the split
form the method runs (a single split of attention per task, then a combine),
so tests can pin it against the monolithic form.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

from persistent_moe_amd import workloads as wlmod


# ---------------------------------------------------------------------------
# elementwise definitions
# ---------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each float64, ties to even (8 significant bits).

    Written from the format's definition: x = m 2**e with m in [1/2, 1); keep
    m to 8 bits with round-half-even (numpy's ``rint``).  Values here are far
    from bf16 overflow and underflow, which are not handled.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 (e4m3fn) codes, from the format's definition.

    Bit 7 is the sign, bits 6-3 the exponent e (bias 7), bits 2-0 the
    mantissa m: e > 0 gives 2**(e - 7) * (1 + m/8), e = 0 the subnormal
    2**-6 * m/8; e = 15 with m = 7 is NaN (the format has no infinities).
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    out = sign * mag
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, out)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain  (the ADD_RMSNORM task's normalisation)."""
    return x / np.sqrt(np.mean(x * x) + eps) * gain


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary position embedding of every head row of ``x`` [H, hd] at ``pos``.

    Rotate-half convention: element i pairs with element i + hd/2, rotated by
    the angle pos * theta**(-2i/hd), i < hd/2.
    """
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


# ---------------------------------------------------------------------------
# attention (ATTN_DECODE / ATTN_COMBINE)
# ---------------------------------------------------------------------------
def attention_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one new token.

    q [Hq, hd]; K, V [n, Hkv, hd] are the visible cached keys and values.
    Query head i reads key/value head floor(i / (Hq/Hkv)); scores are scaled
    by 1/sqrt(hd); no bias, mask or soft-cap.
    """
    Hq, hd = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, hd))
    for i in range(Hq):
        g = i // G
        s = K[:, g, :] @ q[i] / math.sqrt(hd)
        p = softmax(s)
        out[i] = p @ V[:, g, :]
    return out


def attention_split(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Unnormalised partial of one split of keys: (m, l, o) per query head.

    m = max score, l = sum exp(s - m), o = sum exp(s - m) V.
    """
    Hq, hd = q.shape
    G = Hq // K.shape[1]
    m = np.empty(Hq)
    l = np.empty(Hq)
    o = np.empty((Hq, hd))
    for i in range(Hq):
        g = i // G
        s = K[:, g, :] @ q[i] / math.sqrt(hd)
        m[i] = np.max(s)
        e = np.exp(s - m[i])
        l[i] = np.sum(e)
        o[i] = e @ V[:, g, :]
    return m, l, o


def attention_combine(parts) -> np.ndarray:
    """Merge split partials: o = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s."""
    ms = np.stack([p[0] for p in parts])          # [S, Hq]
    M = np.max(ms, axis=0)
    scale = np.exp(ms - M)
    num = sum(scale[s][:, None] * parts[s][2] for s in range(len(parts)))
    den = sum(scale[s] * parts[s][1] for s in range(len(parts)))
    return num / den[:, None]


# ---------------------------------------------------------------------------
# routing and experts (ROUTER_GEMM, ROUTER_TOPK, MoE up-gate / down / combine)
# ---------------------------------------------------------------------------
@dataclass
class Route:
    ids: np.ndarray        # [k] expert ids, highest logit first (ties: lower id first)
    weights: np.ndarray    # [k] softmax probabilities of ids, renormalised to sum 1
    margin: float          # r_(k) - r_(k+1) of the sorted logits (inf if k == E)
    probs: np.ndarray      # [E] full softmax


def route(logits: np.ndarray, k: int) -> Route:
    """Top-k experts by router logit with softmax-renormalised gate weights."""
    E = logits.shape[0]
    order = sorted(range(E), key=lambda e: (-logits[e], e))
    ids = np.array(order[:k], dtype=np.int64)
    p = softmax(logits)
    w = p[ids] / np.sum(p[ids])
    margin = float(logits[order[k - 1]] - logits[order[k]]) if k < E else math.inf
    return Route(ids=ids, weights=w, margin=margin, probs=p)


def swiglu(h: np.ndarray, w_upgate: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SwiGLU FFN: W_down (silu(W_gate h) * (W_up h)); W_upgate = [W_gate; W_up]."""
    inter = w_upgate.shape[0] // 2
    g = w_upgate[:inter] @ h
    u = w_upgate[inter:] @ h
    return w_down @ (silu(g) * u)


def moe(h: np.ndarray, r: Route, expert) -> np.ndarray:
    """sum over the selected experts, in the order of ``r.ids``, of w_e * FFN_e(h)."""
    out = np.zeros_like(h)
    for e, w in zip(r.ids, r.weights):
        w_ug, w_d = expert(int(e))
        out = out + w * swiglu(h, w_ug, w_d)
    return out


# ---------------------------------------------------------------------------
# inputs: weights and cache drawn from the seeded generator
# ---------------------------------------------------------------------------
def _f64(t) -> np.ndarray:
    return t.float().numpy().astype(np.float64)


class Weights:
    """Lazily drawn float64 copies of the bf16 weights of one workload.

    ``cache_limit`` bounds the bytes kept between calls; large tensors (the
    LM head, the embedding table) are streamed in row blocks instead.
    """

    def __init__(self, wl: "wlmod.Workload", cache_limit: int = 1 << 30):
        self.wl = wl
        self.cfg = wl.model
        self.seed = wl.seed
        self.shapes = wlmod.weight_shapes(self.cfg)
        self.cache: Dict[tuple, np.ndarray] = {}
        self.cache_bytes = 0
        self.cache_limit = cache_limit

    def _get(self, key, make):
        if key in self.cache:
            return self.cache[key]
        a = make()
        if self.cache_bytes + a.nbytes <= self.cache_limit:
            self.cache[key] = a
            self.cache_bytes += a.nbytes
        return a

    def layer(self, name: str, layer: int) -> np.ndarray:
        shape = self.shapes[name]
        return self._get((name, layer), lambda: _f64(
            wlmod.gen_tensor(self.seed, name, shape, layer=layer)))

    def expert(self, layer: int, e: int):
        def make(name):
            w = wlmod.gen_tensor(self.seed, name, self.shapes[name], layer=layer, expert=e)
            if not self.cfg.expert_fp8:
                return _f64(w)
            # FP8 storage: the expert computes with s_r * E4M3(q[r, k])
            codes, scale = wlmod.quantize_e4m3_rows(w)
            return e4m3_decode(codes.numpy()) * scale.numpy().astype(np.float64)[:, None]
        ug = self._get(("w_upgate", layer, e), lambda: make("w_upgate"))
        dn = self._get(("w_down", layer, e), lambda: make("w_down"))
        return ug, dn

    def router_bias(self, layer: int) -> Optional[np.ndarray]:
        b = wlmod.router_bias(self.seed, self.cfg, layer)
        return None if b is None else _f64(b)

    def dense_ffn(self, layer: int):
        return self.layer("w_upgate", layer), self.layer("w_down", layer)

    def final_norm(self) -> np.ndarray:
        return self._get(("final_norm",), lambda: _f64(
            wlmod.gen_tensor(self.seed, "final_norm", (self.cfg.d_model,))))

    def embed_row(self, token: int) -> np.ndarray:
        d = self.cfg.d_model
        return _f64(wlmod.gen_tensor(self.seed, "embed", (self.cfg.vocab, d),
                                     rows=slice(token, token + 1)))[0]

    def lm_head_rows(self, r0: int, r1: int) -> np.ndarray:
        name = "embed" if self.cfg.tied_embeddings else "lm_head"
        return _f64(wlmod.gen_tensor(self.seed, name, (self.cfg.vocab, self.cfg.d_model),
                                     rows=slice(r0, r1)))


@dataclass
class Sequence:
    """One sequence's cache: pre-filled positions [0, ctx0) drawn from the
    generator, and float64 copies of every appended (bf16-rounded) entry."""

    seq_id: int
    ctx0: int
    length: int
    appended_k: Dict[int, List[np.ndarray]] = field(default_factory=dict)
    appended_v: Dict[int, List[np.ndarray]] = field(default_factory=dict)
    prefill_cache: Dict[tuple, np.ndarray] = field(default_factory=dict)


def new_sequence(seq_id: int, ctx0: int) -> Sequence:
    return Sequence(seq_id=seq_id, ctx0=ctx0, length=ctx0)


def cached_kv(wl, seq: Sequence, layer: int, p0: int, p1: int, keep: bool = True):
    """K, V [p1-p0, Hkv, hd] of positions [p0, p1) of ``seq`` at ``layer``."""
    cfg = wl.model
    parts_k, parts_v = [], []
    if p0 < seq.ctx0:
        q1 = min(p1, seq.ctx0)
        key = (layer, p0, q1)
        if key in seq.prefill_cache:
            k, v = seq.prefill_cache[key]
        else:
            k = _f64(wlmod.gen_kv(wl.seed, cfg, seq.seq_id, layer, "k", p0, q1))
            v = _f64(wlmod.gen_kv(wl.seed, cfg, seq.seq_id, layer, "v", p0, q1))
            if keep:
                seq.prefill_cache = {kk: vv for kk, vv in seq.prefill_cache.items() if kk[0] != layer}
                seq.prefill_cache[key] = (k, v)
        parts_k.append(k)
        parts_v.append(v)
    if p1 > seq.ctx0:
        a0 = max(p0, seq.ctx0) - seq.ctx0
        a1 = p1 - seq.ctx0
        parts_k.append(np.stack(seq.appended_k[layer][a0:a1]))
        parts_v.append(np.stack(seq.appended_v[layer][a0:a1]))
    return np.concatenate(parts_k), np.concatenate(parts_v)


# ---------------------------------------------------------------------------
# one decode step
# ---------------------------------------------------------------------------
@dataclass
class LayerTaps:
    h: np.ndarray                 # normed input of the attention branch
    q: np.ndarray                 # [Hq, hd] after RoPE
    k_new: np.ndarray             # [Hkv, hd] appended key (bf16 values)
    v_new: np.ndarray
    attn: np.ndarray              # [Hq*hd] attention output before W_o
    attn_out: np.ndarray          # [d] after W_o
    router_logits: Optional[np.ndarray] = None
    route: Optional[Route] = None
    ffn_out: Optional[np.ndarray] = None  # MoE (or dense FFN) output [d]
    x_out: Optional[np.ndarray] = None    # residual after the layer


@dataclass
class StepResult:
    logits: np.ndarray            # [V]
    token: int                    # argmax, ties to the lowest id
    layers: List[LayerTaps]


def _attention_branch(wl, W: Weights, seq: Sequence, layer: int, h: np.ndarray,
                      pos: int, keep_cache: bool) -> LayerTaps:
    cfg = wl.model
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    qkv = W.layer("w_qkv", layer) @ h
    q = qkv[:Hq * hd].reshape(Hq, hd)
    k = qkv[Hq * hd:(Hq + Hkv) * hd].reshape(Hkv, hd)
    v = qkv[(Hq + Hkv) * hd:].reshape(Hkv, hd)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    k_b, v_b = bf16_round(k), bf16_round(v)
    seq.appended_k.setdefault(layer, []).append(k_b)
    seq.appended_v.setdefault(layer, []).append(v_b)
    window = cfg.layer_window(layer)
    lo = max(0, pos - window + 1) if window > 0 else 0
    K, V = cached_kv(wl, seq, layer, lo, pos + 1, keep=keep_cache)
    o = attention_decode(q, K, V).reshape(-1)
    a = W.layer("w_o", layer) @ o
    return LayerTaps(h=h, q=q, k_new=k_b, v_new=v_b, attn=o, attn_out=a)


def decode_one(wl, W: Weights, seq: Sequence, token: int, keep_cache: bool = True,
               lm_rows: int = 16384) -> StepResult:
    """Decode one token of one sequence; appends its K/V to ``seq``."""
    cfg = wl.model
    pos = seq.length
    eps = cfg.rms_eps
    x = W.embed_row(token)
    taps: List[LayerTaps] = []
    for l in range(cfg.n_layers):
        h = rms_norm(x, W.layer("attn_norm", l), eps)
        t = _attention_branch(wl, W, seq, l, h, pos, keep_cache)
        if cfg.parallel_block:
            # x += Attn(RMSNorm(x)) + MoE(RMSNorm(x)) with one shared norm
            if cfg.is_moe:
                r = W.layer("w_router", l) @ h
                bias = W.router_bias(l)
                if bias is not None:
                    # a router bias is part of the logits: it moves both the
                    # selection and the softmax gate weights
                    r = r + bias
                sel = route(r, cfg.top_k)
                m = moe(h, sel, lambda e, l=l: W.expert(l, e))
                t.router_logits, t.route = r, sel
            else:
                m = swiglu(h, *W.dense_ffn(l))
            x = x + t.attn_out + m
        else:
            # sequential pre-norm block: x += Attn(N1(x)); x += FFN(N2(x))
            x = x + t.attn_out
            h2 = rms_norm(x, W.layer("ffn_norm", l), eps)
            m = swiglu(h2, *W.dense_ffn(l))
            x = x + m
        t.ffn_out = m
        t.x_out = x
        taps.append(t)
    seq.length += 1
    hf = rms_norm(x, W.final_norm(), eps)
    logits = np.empty(cfg.vocab)
    for r0 in range(0, cfg.vocab, lm_rows):
        r1 = min(cfg.vocab, r0 + lm_rows)
        logits[r0:r1] = W.lm_head_rows(r0, r1) @ hf
    return StepResult(logits=logits, token=int(np.argmax(logits)), layers=taps)


# ---------------------------------------------------------------------------
# the next token: greedy or temperature sampling after the LM head
# ---------------------------------------------------------------------------
_M32 = 0xFFFFFFFF


def _fmix32(h: np.ndarray) -> np.ndarray:
    """MurmurHash3's 32-bit finaliser (Austin Appleby), elementwise on uint64
    arrays holding 32-bit values: xor-shift 16, multiply 0x85ebca6b, xor-shift
    13, multiply 0xc2b2ae35, xor-shift 16, all modulo 2**32."""
    h = np.asarray(h, dtype=np.uint64) & np.uint64(_M32)
    h ^= h >> np.uint64(16)
    h = (h * np.uint64(0x85EBCA6B)) & np.uint64(_M32)
    h ^= h >> np.uint64(13)
    h = (h * np.uint64(0xC2B2AE35)) & np.uint64(_M32)
    h ^= h >> np.uint64(16)
    return h


def sampling_uniforms(seed: int, position: int, slot: int, n: int) -> np.ndarray:
    """One uniform in (0, 1) per vocabulary id for the token sampled at cache
    position ``position`` of batch slot ``slot``: a counter-based stream,
    u_v = (floor(h_v / 2**8) + 1/2) / 2**24 (24 bits, so the value is exact
    in single precision) with
    h_v = fmix32(fmix32(fmix32(fmix32(seed) ^ position) ^ slot) ^ v)."""
    k = _fmix32(np.array([seed & _M32]))[0]
    k = _fmix32(np.array([int(k) ^ (position & _M32)]))[0]
    k = _fmix32(np.array([int(k) ^ (slot & _M32)]))[0]
    h = _fmix32(np.arange(n, dtype=np.uint64) ^ np.uint64(k))
    return ((h >> np.uint64(8)).astype(np.float64) + 0.5) / 16777216.0


def sample_token(logits: np.ndarray, temperature: float, seed: int = 0, position: int = 0,
                 slot: int = 0) -> Tuple[int, float]:
    """The next token and the margin of the decision.

    temperature == 0: greedy, the largest logit (ties to the lowest id).
    temperature > 0: a draw from softmax(logits / temperature) by the
    Gumbel-max method: the id maximising logits_v / T + g_v, with the Gumbel
    noise g_v = -ln(-ln u_v) of the counter-based uniforms above (ties to the
    lowest id).  The margin is the gap between the best and the second-best
    score (a near-tie can go either way under rounding).
    """
    z = np.asarray(logits, dtype=np.float64)
    if temperature > 0:
        u = sampling_uniforms(seed, position, slot, z.shape[0])
        z = z / temperature - np.log(-np.log(u))
    tok = int(np.argmax(z))
    if z.shape[0] > 1:
        top2 = np.partition(z, -2)[-2:]
        gap = float(top2[1] - top2[0])
    else:
        gap = math.inf
    return tok, gap


def decode_step(wl, W: Weights, seqs: List[Sequence], tokens: List[int],
                keep_cache: bool = True) -> List[StepResult]:
    """One decode step of a batch: each sequence independently."""
    return [decode_one(wl, W, s, t, keep_cache) for s, t in zip(seqs, tokens)]


def greedy_decode(wl, steps: int, W: Optional[Weights] = None) -> Tuple[List[List[int]], List[List[StepResult]]]:
    """Greedy decode of a fixed-length batch (no swaps) from the seeded start.

    Returns the fed tokens per step and the step results.
    """
    W = W or Weights(wl)
    plan = wlmod.plan_batch(wl, steps)
    seqs = [new_sequence(plan.slots[b][0][1].seq_id, plan.slots[b][0][1].ctx) for b in range(wl.batch)]
    toks = [plan.slots[b][0][1].token for b in range(wl.batch)]
    fed, results = [], []
    for _ in range(steps):
        fed.append(list(toks))
        res = decode_step(wl, W, seqs, toks)
        results.append(res)
        toks = [r.token for r in res]
    return fed, results
