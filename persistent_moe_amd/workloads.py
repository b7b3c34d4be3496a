"""Workload definitions and the seeded, element-addressable input generator.

This module holds the shapes of the five decode workloads and the recipe that
turns a seed into every input of a decode step: weights, norm gains,
embeddings, the pre-filled KV cache, start tokens, context lengths and block
tables.  It contains none of the decode arithmetic.  Both the CPU oracle and
the GPU harness draw their inputs from here, so the two sides see bit-identical
inputs without sharing any code that computes the method.

Model family (the persistent decode megakernel pages, "One kernel for the full
decode step" and the 16-task-type list): a parallel-block MoE transformer,
x += Attn(RMSNorm(x)) + MoE(RMSNorm(x)), plus a sequential pre-norm dense
decoder shaped like Llama-3.2-1B for the dense opcodes.

Generator (counter based, so any slice of any tensor can be produced alone):

* ``fmix32`` is the 32-bit finaliser of MurmurHash3 (Austin Appleby, public
  domain): xor-shift 16, multiply 0x85ebca6b, xor-shift 13, multiply
  0xc2b2ae35, xor-shift 16, all modulo 2**32.
* A tensor gets a 32-bit key from (seed, crc32(name), layer, expert).
* Element ``i`` (a 64-bit flat index) yields two words
  ``h_j = fmix32(lo ^ fmix32(hi ^ k_j))`` for two stream keys ``k_1, k_2``,
  which become uniforms ``u_j = (h_j + 0.5) / 2**32``.
* Box-Muller in float64: ``z = sqrt(-2 ln u_1) cos(2 pi u_2)``; the value
  ``mean + std * z`` is rounded to float32 and then to bfloat16, both
  round-to-nearest-even.

All integer work is done in int64 with every intermediate below 2**63, so the
same code gives the same bits on the CPU and on the GPU.
"""
from __future__ import annotations

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

M32 = 0xFFFFFFFF


# ----------------------------------------------------------------------------
# model shapes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelConfig:
    """Shape of one decoder.  ``n_experts == 0`` means a dense SwiGLU FFN."""

    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    n_experts: int = 0
    top_k: int = 0
    expert_inter: int = 0
    ffn_inter: int = 0
    tied_embeddings: bool = False
    parallel_block: bool = True
    page_size: int = 16
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-5
    swa_window: int = 0        # 0: every layer attends to the whole context
    swa_period: int = 0        # layer l is global iff l % swa_period == swa_period - 1
    router_zipf: float = 0.0   # > 0: each layer's router has a bias that skews routing (router_bias)
    expert_fp8: bool = False   # expert weights stored as E4M3 codes with a per-row scale (quantize_e4m3_rows)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def attn_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def layer_window(self, layer: int) -> int:
        """Number of most recent keys layer ``layer`` may attend to (0 = all)."""
        if self.swa_window <= 0 or self.swa_period <= 0:
            return 0
        if layer % self.swa_period == self.swa_period - 1:
            return 0
        return self.swa_window


@dataclass(frozen=True)
class Workload:
    """A decode workload: a model, a batch, its starting contexts and steps."""

    name: str
    model: ModelConfig
    batch: int
    ctx: str                   # "fixed:<n>", "loguniform:<lo>:<hi>" or "list:<n0>,<n1>,..." (per sequence id)
    steps: int
    seed: int
    swap_every: int = 0        # continuous batching: replace one sequence every N steps
    page_slack: int = 0        # extra free pages in the pool

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY_MOE = ModelConfig(
    name="tiny-moe", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=1, head_dim=64,
    vocab=1024, n_experts=8, top_k=2, expert_inter=128, tied_embeddings=False,
    parallel_block=True)

DENSE_1B = ModelConfig(
    name="dense-llama1b-shape", n_layers=16, d_model=2048, n_q_heads=32, n_kv_heads=8,
    head_dim=64, vocab=128256, ffn_inter=8192, tied_embeddings=True, parallel_block=False)

MOE_30B = ModelConfig(
    name="moe-30b-a3.3b", n_layers=48, d_model=2048, n_q_heads=32, n_kv_heads=4,
    head_dim=128, vocab=256000, n_experts=128, top_k=8, expert_inter=768,
    tied_embeddings=False, parallel_block=True)

MOE_30B_SWA = replace(MOE_30B, name="moe-30b-a3.3b-swa", swa_window=4096, swa_period=4)
MOE_30B_ZIPF = replace(MOE_30B, name="moe-30b-a3.3b-zipf", router_zipf=1.2)
MOE_30B_FP8 = replace(MOE_30B, name="moe-30b-a3.3b-fp8-experts", expert_fp8=True)

WORKLOADS = {
    "tiny": Workload("tiny-moe-bs1-ctx64", TINY_MOE, batch=1, ctx="fixed:64", steps=8, seed=0),
    "dense1b": Workload("dense1b-bs1-ctx4k", DENSE_1B, batch=1, ctx="fixed:4096", steps=128, seed=1),
    "moe30b": Workload("moe30b-bs1-ctx8k", MOE_30B, batch=1, ctx="fixed:8192", steps=256, seed=2),
    "moe30b_bs8": Workload("moe30b-bs8-ragged", MOE_30B, batch=8, ctx="loguniform:512:16384",
                           steps=256, seed=3, swap_every=32),
    "moe30b_256k": Workload("moe30b-bs1-ctx256k-swa", MOE_30B_SWA, batch=1, ctx="fixed:262144",
                            steps=64, seed=4),
    # concentrated routing: the continuous-batching workload with a router
    # bias that favours a seeded few experts per layer (Zipf ranks)
    "moe30b_bs8_zipf": Workload("moe30b-bs8-ragged-zipf", MOE_30B_ZIPF, batch=8, ctx="loguniform:512:16384",
                                steps=256, seed=5, swap_every=32),
    # the bs=1 8K workload (same seed, so the same bf16 draws) with the expert
    # weights streamed as FP8
    "moe30b_fp8": Workload("moe30b-bs1-ctx8k-fp8", MOE_30B_FP8, batch=1, ctx="fixed:8192", steps=256, seed=2),
    # and the continuous-batching bs=8 workload (same seed as moe30b_bs8)
    "moe30b_bs8_fp8": Workload("moe30b-bs8-ragged-fp8", MOE_30B_FP8, batch=8, ctx="loguniform:512:16384",
                               steps=256, seed=3, swap_every=32),
}


# ----------------------------------------------------------------------------
# counter-based generator
# ----------------------------------------------------------------------------
def fmix32_int(h: int) -> int:
    """MurmurHash3 32-bit finaliser on a Python int."""
    h &= M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & M32
    h ^= h >> 16
    return h


def tensor_key(seed: int, name: str, layer: int = -1, expert: int = -1) -> int:
    k = fmix32_int(seed * 0x9E3779B9 + 0x51ED270B)
    k = fmix32_int(k ^ zlib.crc32(name.encode()))
    k = fmix32_int(k ^ ((layer + 1) * 0x85EBCA77))
    k = fmix32_int(k ^ ((expert + 1) * 0xC2B2AE3D))
    return k


class _NumpyOps:
    """uint64 numpy arrays; products wrap modulo 2**64 and are masked to 32 bits."""

    @staticmethod
    def arange(start, count):
        return np.arange(start, start + count, dtype=np.uint64)

    @staticmethod
    def mul32(a, c):
        return (a * np.uint64(c)) & np.uint64(M32)

    @staticmethod
    def f64(a):
        return a.astype(np.float64)

    frexp = staticmethod(np.frexp)
    sqrt = staticmethod(np.sqrt)
    where = staticmethod(np.where)

    @staticmethod
    def f32_bits(x64):
        return x64.astype(np.float32).view(np.uint32).astype(np.uint64)


class _TorchOps:
    """int64 tensors; a 32x32-bit product is split in 16-bit halves to stay < 2**63."""

    def __init__(self, device):
        self.device = device

    def arange(self, start, count):
        return torch.arange(start, start + count, dtype=torch.int64, device=self.device)

    @staticmethod
    def mul32(a, c):
        lo, hi = c & 0xFFFF, c >> 16
        return (a * lo + (((a * hi) & 0xFFFF) << 16)) & M32

    @staticmethod
    def f64(a):
        return a.to(torch.float64)

    @staticmethod
    def frexp(x):
        m, e = torch.frexp(x)
        return m, e.to(torch.float64)

    sqrt = staticmethod(torch.sqrt)
    where = staticmethod(torch.where)

    @staticmethod
    def f32_bits(x64):
        return x64.to(torch.float32).view(torch.int32).to(torch.int64) & M32


def _fmix32(h, ops):
    h = h ^ (h >> 16)
    h = ops.mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = ops.mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _words(key: int, start: int, count: int, ops):
    idx = ops.arange(start, count)
    lo = idx & M32
    hi = idx >> 32
    h1 = _fmix32(lo ^ _fmix32(hi ^ fmix32_int(key ^ 0x68E31DA4), ops), ops)
    h2 = _fmix32(lo ^ _fmix32(hi ^ fmix32_int(key ^ 0xB5297A4D), ops), ops)
    return h1, h2


_LN2 = 0.6931471805599453
_PI_4 = 0.7853981633974483
_SQRT2 = 1.4142135623730951
_LOG_C = [1.0 / (2 * k + 1) for k in range(11)]            # atanh series of ln
_COS_C = [(-1.0) ** j / math.factorial(2 * j) for j in range(10)]
_SIN_C = [(-1.0) ** j / math.factorial(2 * j + 1) for j in range(10)]


def _neg2_ln_u(h1, ops):
    """-2 ln u with u = (h1 + 1/2) / 2**32, from +, -, *, / and frexp only.

    u = n / 2**33 with n = 2 h1 + 1 exact in float64.  n = m 2**e with m in
    [sqrt(1/2), sqrt(2)), and ln m = 2 atanh(s), s = (m - 1)/(m + 1), summed
    as 2 s sum_k s**(2k) / (2k + 1) for k <= 10 (|s| < 0.172, error < 1e-17).
    """
    n = ops.f64(h1) * 2.0 + 1.0
    m, e = ops.frexp(n)                 # n = m 2**e, m in [1/2, 1)
    m = m * 2.0
    e = e - 1.0
    big = m > _SQRT2
    m = ops.where(big, m * 0.5, m)
    e = ops.where(big, e + 1.0, e)
    s = (m - 1.0) / (m + 1.0)
    t = s * s
    acc = t * 0.0 + _LOG_C[10]
    for k in range(9, -1, -1):
        acc = acc * t + _LOG_C[k]
    ln_u = (e - 33.0) * _LN2 + 2.0 * s * acc
    return -2.0 * ln_u


def _cos_2pi_u(h2, ops):
    """cos(2 pi u) with u = (h2 + 1/2) / 2**32, from +, -, * only.

    The top three bits of h2 give the octant q; the rest give r in (0, 1), so
    2 pi u = q pi/4 + r pi/4 exactly.  Odd octants are written as the next
    quadrant minus (1 - r) pi/4, leaving |a| <= pi/4 for the Taylor series
    (ten terms each for sin and cos, error < 1e-17).
    """
    q = h2 >> 29
    rem = ops.f64(h2 & 0x1FFFFFFF) * 2.0 + 1.0          # odd, < 2**30
    r = rem * (1.0 / 1073741824.0)
    odd = (q & 1) == 1
    a = ops.where(odd, -((1.0 - r) * _PI_4), r * _PI_4)
    quad = ((q + 1) >> 1) & 3
    t = a * a
    c = t * 0.0 + _COS_C[9]
    sn = t * 0.0 + _SIN_C[9]
    for j in range(8, -1, -1):
        c = c * t + _COS_C[j]
        sn = sn * t + _SIN_C[j]
    sn = sn * a
    out = ops.where(quad == 0, c, -sn)
    out = ops.where(quad == 2, -c, out)
    out = ops.where(quad == 3, sn, out)
    return out


def _bf16_bits(x64, ops):
    """float64 -> float32 -> bfloat16, both round-to-nearest-even; 16-bit codes."""
    b = ops.f32_bits(x64)
    return (b + 0x7FFF + ((b >> 16) & 1)) >> 16


def normal_bf16_codes(key: int, start: int, count: int, mean: float, std: float, ops):
    h1, h2 = _words(key, start, count, ops)
    z = ops.sqrt(_neg2_ln_u(h1, ops)) * _cos_2pi_u(h2, ops)
    return _bf16_bits(z * std + mean, ops)


_GEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gen")
_clib = None


def _host_lib():
    """The C transcription of this generator (gen/pmgen.c), if it is built."""
    global _clib
    if _clib is None:
        import ctypes
        path = os.path.join(_GEN_DIR, "libpmgen.so")
        if not os.path.exists(path):
            _clib = False
            return None
        lib = ctypes.CDLL(path)
        lib.pmgen_normal_bf16.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.pmgen_set_coef.argtypes = [ctypes.c_void_p] * 3
        coef = [np.array(c, dtype=np.float64) for c in (_LOG_C, _COS_C, _SIN_C)]
        lib.pmgen_set_coef(*[c.ctypes.data for c in coef])
        _clib = lib
    return _clib or None


def normal_bf16(key: int, start: int, count: int, mean: float, std: float,
                device="cpu", backend: str = "auto") -> torch.Tensor:
    """Elements [start, start+count) of the N(mean, std^2) stream ``key`` as bf16.

    ``backend``: "auto" (C on the host when built, torch on a GPU), "numpy",
    "c" or "torch"; all give the same bits.
    """
    dev = torch.device(device)
    if dev.type == "cpu" and backend in ("auto", "c") and _host_lib() is not None:
        out = np.empty(count, dtype=np.uint16)
        _host_lib().pmgen_normal_bf16(key & M32, start, count, mean, std, out.ctypes.data)
        return torch.from_numpy(out.view(np.int16)).view(torch.bfloat16)
    if dev.type == "cpu" and backend != "torch":
        if backend == "c":
            raise RuntimeError("libpmgen.so is not built")
        codes = normal_bf16_codes(key, start, count, mean, std, _NumpyOps)
        return torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    codes = normal_bf16_codes(key, start, count, mean, std, _TorchOps(dev))
    codes = torch.where(codes >= 32768, codes - 65536, codes)
    return codes.to(torch.int16).view(torch.bfloat16)


def uniform_f64(key: int, start: int, count: int) -> np.ndarray:
    h1, _ = _words(key, start, count, _NumpyOps)
    return (h1.astype(np.float64) + 0.5) * (1.0 / 4294967296.0)


def fill_normal_(out: torch.Tensor, key: int, mean: float, std: float,
                 start: int = 0, chunk: int = 0) -> torch.Tensor:
    """Fill a contiguous bf16 tensor with elements [start, start+numel) of a stream."""
    flat = out.view(-1)
    n = flat.numel()
    if out.device.type == "cpu":
        chunk = chunk or (1 << 22)
        spans = [(s, min(chunk, n - s)) for s in range(0, n, chunk)]

        def work(sp):
            s, c = sp
            flat[s:s + c] = normal_bf16(key, start + s, c, mean, std)

        if len(spans) > 1:
            with ThreadPoolExecutor(max_workers=_cpu_threads()) as ex:
                list(ex.map(work, spans))
        elif spans:
            work(spans[0])
        return out
    chunk = chunk or (1 << 25)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        flat[s:s + c] = normal_bf16(key, start + s, c, mean, std, device=out.device)
    return out


def fill_normal_keyed_(out: torch.Tensor, keys: List[int], mean: float, std: float,
                       group_elems: int = 1 << 25, backend: str = "auto") -> torch.Tensor:
    """Fill out[i] (contiguous, bf16) with elements [0, numel/len(keys)) of
    stream keys[i], for each leading index i.  On a GPU several streams are
    drawn in one vectorised pass; the bits equal those of ``fill_normal_``."""
    n_keys = out.shape[0]
    assert n_keys == len(keys)
    per = out[0].numel()
    assert per < (1 << 32)
    if out.device.type == "cpu" and backend != "torch":
        for i, k in enumerate(keys):
            fill_normal_(out[i], k, mean, std)
        return out
    ops = _TorchOps(out.device)
    flat = out.view(n_keys, per)
    # element i of stream k: h_j = fmix32(i ^ fmix32(0 ^ k_j)), as in _words with hi = 0
    m1 = [fmix32_int(fmix32_int(k ^ 0x68E31DA4)) for k in keys]
    m2 = [fmix32_int(fmix32_int(k ^ 0xB5297A4D)) for k in keys]
    per_chunk = max(1, min(per, group_elems))
    kpg = max(1, group_elems // per) if per <= group_elems else 1
    for k0 in range(0, n_keys, kpg):
        k1 = min(n_keys, k0 + kpg)
        for s in range(0, per, per_chunk):
            c = min(per_chunk, per - s)
            idx = torch.arange(s, s + c, dtype=torch.int64, device=out.device)
            idx = idx.unsqueeze(0).expand(k1 - k0, c)
            a1 = torch.tensor(m1[k0:k1], dtype=torch.int64, device=out.device).unsqueeze(1)
            a2 = torch.tensor(m2[k0:k1], dtype=torch.int64, device=out.device).unsqueeze(1)
            h1 = _fmix32(idx ^ a1, ops)
            h2 = _fmix32(idx ^ a2, ops)
            z = ops.sqrt(_neg2_ln_u(h1, ops)) * _cos_2pi_u(h2, ops)
            codes = _bf16_bits(z * std + mean, ops)
            codes = torch.where(codes >= 32768, codes - 65536, codes)
            flat[k0:k1, s:s + c] = codes.to(torch.int16).view(torch.bfloat16)
    return out


def _cpu_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


# ----------------------------------------------------------------------------
# what each tensor is drawn from
# ----------------------------------------------------------------------------
W_STD = 0.02          # projection weights N(0, 0.02)
GAIN_MEAN, GAIN_STD = 1.0, 0.1   # RMSNorm gains 1 + N(0, 0.1)
EMB_STD = 1.0         # embeddings N(0, 1)
KV_STD = 1.0          # pre-filled KV N(0, 1)


def weight_shapes(cfg: ModelConfig) -> dict:
    """Per-layer tensor shapes, row-major [out, in] for projections."""
    d, I = cfg.d_model, cfg.expert_inter
    s = {
        "attn_norm": (d,),
        "w_qkv": (cfg.qkv_rows, d),
        "w_o": (d, cfg.attn_dim),
    }
    if cfg.is_moe:
        s["w_router"] = (cfg.n_experts, d)
        s["w_upgate"] = (2 * I, d)     # per expert; gate rows first, then up rows
        s["w_down"] = (d, I)           # per expert
    else:
        s["ffn_norm"] = (d,)
        s["w_upgate"] = (2 * cfg.ffn_inter, d)
        s["w_down"] = (d, cfg.ffn_inter)
    return s


def tensor_dist(name: str):
    if name in ("attn_norm", "ffn_norm", "final_norm"):
        return GAIN_MEAN, GAIN_STD
    if name == "embed":
        return 0.0, EMB_STD
    return 0.0, W_STD


def gen_tensor(seed: int, name: str, shape, layer: int = -1, expert: int = -1,
               device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """A whole tensor (or a row slice of a 2-D one) as bf16."""
    mean, std = tensor_dist(name)
    key = tensor_key(seed, name, layer, expert)
    if rows is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        return fill_normal_(out, key, mean, std)
    r0, r1 = rows.start or 0, rows.stop if rows.stop is not None else shape[0]
    ncol = int(np.prod(shape[1:]))
    out = torch.empty((r1 - r0,) + tuple(shape[1:]), dtype=torch.bfloat16, device=device)
    return fill_normal_(out, key, mean, std, start=r0 * ncol)


def router_bias(seed: int, cfg: ModelConfig, layer: int) -> Optional[torch.Tensor]:
    """The router bias of one layer as bf16 [E], or None without one.

    Experts get Zipf ranks from a seeded permutation per layer; expert e of
    rank k (0-based) has bias -s * ln(k + 1), s = cfg.router_zipf, so that
    with the bias alone routing picks expert ranks with weights proportional
    to (k + 1)**-s (real traffic concentrates on a few experts).  Rounded to
    float32 and then bf16, both round-to-nearest-even, like every weight.
    """
    if cfg.router_zipf <= 0 or cfg.n_experts == 0:
        return None
    rank = np.empty(cfg.n_experts, dtype=np.int64)
    rank[permutation(seed, "router_rank_layer%d" % layer, cfg.n_experts)] = np.arange(cfg.n_experts)
    b = -cfg.router_zipf * np.log(rank.astype(np.float64) + 1.0)
    return torch.from_numpy(b.astype(np.float32)).to(torch.bfloat16)


E4M3_MAX = 448.0      # the largest finite OCP E4M3 (e4m3fn) value
# 1/448 rounded to float32: the row scale is amax times this (one float32
# multiply, the same bits on any device)
INV_E4M3_MAX_F32 = float(np.float32(1.0 / 448.0))


def _pow2_f64(n: torch.Tensor) -> torch.Tensor:
    """2.0 ** n for integer tensors n in [-1022, 1023], built from the bits."""
    return ((n.to(torch.int64) + 1023) << 52).view(torch.float64)


def quantize_e4m3_rows(w: torch.Tensor):
    """Per-row FP8 storage of a weight matrix [..., rows, K] (bf16 or float).

    Each row r gets the scale s_r = float32(max_k |w[r, k]| * float32(1/448))
    (1 for an all-zero row) and the codes q[r, k] = E4M3(w[r, k] / s_r): the
    quotient in float64, rounded to the nearest value of the E4M3 grid, ties
    to even, saturating at 448.  Returns (codes as uint8, scales as float32).

    Every operation is exact or correctly rounded (a float32 multiply, a
    float64 divide, frexp, round-half-even after a power-of-two scaling,
    integer bit assembly), so a CPU and a GPU produce the same bits; torch's
    own float8 conversion and its divide-by-scalar are not used, since on a
    GPU they may take hardware or reciprocal paths.
    """
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax * INV_E4M3_MAX_F32, torch.ones_like(amax))
    y = w.double() / scale.double().unsqueeze(-1)
    a = y.abs()
    # binade of a (a = m 2^e, m in [0.5, 1)), at least -6: below 2^-6 the
    # subnormal step 2^-9 applies; three mantissa bits give a step of 2^(eb-3)
    _, e = torch.frexp(a)
    eb = torch.clamp(e.to(torch.int64) - 1, min=-6)
    k = torch.round(a * _pow2_f64(3 - eb)).to(torch.int64)   # a in steps: 8..16 in a binade, 0..8 below
    up = k == 16                                              # rounded up into the next binade
    eb = torch.where(up, eb + 1, eb)
    k = torch.where(up, torch.full_like(k, 8), k)
    normal = k >= 8
    ef = torch.where(normal, eb + 7, torch.zeros_like(eb))     # biased exponent field
    mf = torch.where(normal, k - 8, k)                          # mantissa field
    sat = (ef > 15) | ((ef == 15) & (mf == 7))                  # beyond 448: saturate
    ef = torch.where(sat, torch.full_like(ef, 15), ef)
    mf = torch.where(sat, torch.full_like(mf, 6), mf)
    code = (torch.signbit(y).to(torch.int64) << 7) | (ef << 3) | mf
    return code.to(torch.uint8), scale


def kv_key(seed: int, seq_id: int, layer: int, which: str) -> int:
    return tensor_key(seed, "kv_" + which + "_seq%d" % seq_id, layer)


def gen_kv(seed: int, cfg: ModelConfig, seq_id: int, layer: int, which: str,
           p0: int, p1: int, device="cpu") -> torch.Tensor:
    """Pre-filled K or V of positions [p0, p1) as bf16 [p1-p0, Hkv, hd]."""
    per_pos = cfg.n_kv_heads * cfg.head_dim
    out = torch.empty((p1 - p0, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=device)
    return fill_normal_(out, kv_key(seed, seq_id, layer, which), 0.0, KV_STD, start=p0 * per_pos)


# ----------------------------------------------------------------------------
# per-sequence starting state
# ----------------------------------------------------------------------------
def start_token(seed: int, seq_id: int, vocab: int) -> int:
    u = float(uniform_f64(tensor_key(seed, "start_token", seq_id), 0, 1)[0])
    return min(int(u * vocab), vocab - 1)


def context_length(wl: Workload, seq_id: int) -> int:
    kind, *args = wl.ctx.split(":")
    if kind == "fixed":
        return int(args[0])
    if kind == "list":
        vals = [int(v) for v in args[0].split(",")]
        return vals[seq_id % len(vals)]
    if kind == "loguniform":
        lo, hi = float(args[0]), float(args[1])
        u = float(uniform_f64(tensor_key(wl.seed, "ctx_len", seq_id), 0, 1)[0])
        return int(math.floor(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
    raise ValueError(wl.ctx)


def permutation(seed: int, name: str, n: int) -> np.ndarray:
    """A seeded permutation of range(n): argsort of hash words (ties by index)."""
    h1, _ = _words(tensor_key(seed, name), 0, n, _NumpyOps)
    return np.argsort(h1, kind="stable").astype(np.int64)


@dataclass
class SequenceSlot:
    seq_id: int        # identity of the sequence (selects its KV stream and token)
    ctx: int           # tokens already in the cache before the first step
    token: int         # token fed at the first step


@dataclass
class BatchPlan:
    """Sequences of each batch slot over the run, and the page pool layout."""

    workload: Workload
    slots: List[List[tuple]] = field(default_factory=list)  # per slot: [(first_step, SequenceSlot)]
    num_pages: int = 0
    max_blocks: int = 0
    page_perm: Optional[np.ndarray] = None

    def sequence_at(self, slot: int, step: int) -> tuple:
        """(first_step, SequenceSlot) live in ``slot`` at ``step``."""
        cur = None
        for first, seq in self.slots[slot]:
            if first <= step:
                cur = (first, seq)
        return cur


def plan_batch(wl: Workload, steps: Optional[int] = None) -> BatchPlan:
    """Which sequence occupies each slot at each step, and how many pages exist.

    A slot is refilled every ``swap_every`` steps, one slot at a time in turn
    (slot (s/swap_every - 1) mod B at step s).  Every sequence owns
    ceil((ctx + remaining steps) / page) pages drawn from one pool whose page
    ids are a seeded permutation.
    """
    steps = wl.steps if steps is None else steps
    B = wl.batch
    plan = BatchPlan(workload=wl)
    next_id = 0
    plan.slots = [[] for _ in range(B)]
    for b in range(B):
        plan.slots[b].append((0, _new_seq(wl, next_id)))
        next_id += 1
    if wl.swap_every > 0:
        for s in range(wl.swap_every, steps, wl.swap_every):
            b = (s // wl.swap_every - 1) % B
            plan.slots[b].append((s, _new_seq(wl, next_id)))
            next_id += 1
    ps = wl.model.page_size
    total, maxb = 0, 0
    for b in range(B):
        segs = plan.slots[b]
        for i, (first, seq) in enumerate(segs):
            last = segs[i + 1][0] if i + 1 < len(segs) else steps
            need = -(-(seq.ctx + (last - first)) // ps)
            total += need
            maxb = max(maxb, need)
    plan.num_pages = total + wl.page_slack
    plan.max_blocks = maxb
    plan.page_perm = permutation(wl.seed, "page_pool", plan.num_pages)
    return plan


def _new_seq(wl: Workload, seq_id: int) -> SequenceSlot:
    return SequenceSlot(seq_id=seq_id, ctx=context_length(wl, seq_id),
                        token=start_token(wl.seed, seq_id, wl.model.vocab))


def page_table(plan: BatchPlan, steps: Optional[int] = None) -> dict:
    """Physical pages of every sequence: {seq_id: np.ndarray of page ids}."""
    wl = plan.workload
    steps = wl.steps if steps is None else steps
    ps = wl.model.page_size
    out, cursor = {}, 0
    for b in range(wl.batch):
        segs = plan.slots[b]
        for i, (first, seq) in enumerate(segs):
            last = segs[i + 1][0] if i + 1 < len(segs) else steps
            need = -(-(seq.ctx + (last - first)) // ps)
            out[seq.seq_id] = plan.page_perm[cursor:cursor + need].copy()
            cursor += need
    return out
