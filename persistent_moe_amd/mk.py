"""ctypes binding of libmk.so (include/mk.h), with the same function names.

Argument marshalling only: every step of the decode path runs in the HIP
library.  Loading fails loudly (``MkError``) when the library is not built;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmk.so")

MK_OK = 0
MK_E_INVAL = -1
MK_E_UNSUPPORTED = -2
MK_E_NOMEM = -3
MK_E_HIP = -4
MK_E_TIMEOUT = -5
MK_E_DEVICE = -6
MK_E_STATE = -7

OPCODES = [
    "ADD_RMSNORM", "QKV_PROJ", "O_PROJ", "FFN_UPGATE_ACT", "FFN_DOWN", "LM_HEAD",
    "ATTN_DECODE", "ATTN_COMBINE", "ATTN_DRAIN", "ROUTER_GEMM", "ROUTER_TOPK",
    "ROUTE_FINALIZE", "MOE_GATHER", "MOE_UPGATE_ACT_DRAIN", "MOE_DOWN_DRAIN", "MOE_COMBINE",
]
MK_WAIT_SPLITS = -2
ORDER = {"tuned": 0, "interleaved": 1, "attention_first": 2, "partitioned": 3}
LAUNCH = {"persistent": 0, "per_opcode": 1}
TAPS = {"x": 0, "xn": 1, "qkv": 2, "attn": 3, "router_logits": 4, "topk_ids": 5, "topk_weights": 6,
        "ffn_out": 7, "attn_out": 8, "trace": 9}
EXPORTS = ["mk_workspace_size", "mk_init", "mk_init_noalloc", "mk_build_schedule", "mk_decode_step",
           "mk_decode_step_sample",
           "mk_get_status", "mk_tap_offset", "mk_plan_schedule", "mk_plan_simulate", "mk_destroy", "mk_strerror"]
MK_SAMPLE_ADVANCE = 1


class MkError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code) if _lib else code} ({code})")


class mk_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "vocab", "n_experts", "top_k",
        "expert_inter", "ffn_inter", "parallel_block", "page_size", "max_batch", "swa_window",
        "swa_period")] + [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                          ("expert_fp8", ctypes.c_int32)]


class mk_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "attn_norm", "ffn_norm", "w_qkv", "w_o", "w_router", "w_upgate", "w_down", "router_bias",
        "upgate_scale", "down_scale")]


class mk_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("layers", ctypes.POINTER(mk_layer_weights))]


class mk_kv_pool(ctypes.Structure):
    _fields_ = [("k", ctypes.POINTER(ctypes.c_void_p)), ("v", ctypes.POINTER(ctypes.c_void_p)),
                ("num_pages", ctypes.c_int32)]


class mk_sched_opts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "wave_order", "launch_mode", "attn_split", "n_workgroups", "timeout_ms", "flags",
        "moe_ug_pairs", "moe_dn_rows")]


class mk_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("seed", ctypes.c_uint32), ("flags", ctypes.c_int32)]


class mk_status(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("code", "task", "counter", "value", "target", "workgroup")]


class mk_task(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "op", "layer", "wait_ctr", "wait_target", "signal_ctr", "flags", "n0", "n1", "k0", "k1",
        "group", "batch", "split", "queue")] + [("aux", ctypes.c_int32 * 18)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load(path: Optional[str] = None):
    """Load libmk.so (once).  Raises MkError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise MkError(MK_E_STATE, f"libmk.so not found at {p}; run persistent_moe_amd.build")
    L = ctypes.CDLL(p)
    P = ctypes.c_void_p
    L.mk_workspace_size.argtypes = [ctypes.POINTER(mk_config), ctypes.c_int32]
    L.mk_workspace_size.restype = ctypes.c_size_t
    L.mk_init.argtypes = [ctypes.POINTER(mk_config), ctypes.POINTER(mk_weights), ctypes.POINTER(mk_kv_pool),
                          P, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(P)]
    L.mk_init_noalloc.argtypes = [ctypes.POINTER(mk_config), ctypes.POINTER(mk_weights),
                                  ctypes.POINTER(mk_kv_pool), ctypes.c_int32, ctypes.POINTER(P)]
    L.mk_build_schedule.argtypes = [P, ctypes.c_int32, ctypes.POINTER(mk_sched_opts)]
    L.mk_decode_step.argtypes = [P, P, P, P, P, P, P]
    L.mk_decode_step_sample.argtypes = [P, P, P, P, P, P, ctypes.POINTER(mk_sampling), P, P]
    L.mk_get_status.argtypes = [P, ctypes.POINTER(mk_status)]
    L.mk_tap_offset.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                ctypes.POINTER(ctypes.c_size_t)]
    L.mk_plan_schedule.argtypes = [ctypes.POINTER(mk_config), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(mk_sched_opts), ctypes.c_int32, ctypes.POINTER(mk_task),
                                   ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32)]
    L.mk_plan_simulate.argtypes = [ctypes.POINTER(mk_config), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(mk_sched_opts), ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32)]
    L.mk_destroy.argtypes = [P]
    L.mk_destroy.restype = None
    L.mk_strerror.argtypes = [ctypes.c_int]
    L.mk_strerror.restype = ctypes.c_char_p
    for name in ("mk_init", "mk_init_noalloc", "mk_build_schedule", "mk_decode_step", "mk_decode_step_sample", "mk_get_status",
                 "mk_tap_offset",
                 "mk_plan_schedule", "mk_plan_simulate"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int, what: str) -> int:
    if rc != MK_OK:
        raise MkError(rc, what)
    return rc


def strerror(code: int) -> str:
    return load().mk_strerror(code).decode()


def make_config(model, max_batch: int) -> mk_config:
    """mk_config from a workloads.ModelConfig."""
    return mk_config(
        n_layers=model.n_layers, d_model=model.d_model, n_q_heads=model.n_q_heads,
        n_kv_heads=model.n_kv_heads, head_dim=model.head_dim, vocab=model.vocab,
        n_experts=model.n_experts, top_k=model.top_k, expert_inter=model.expert_inter,
        ffn_inter=model.ffn_inter, parallel_block=int(model.parallel_block), page_size=model.page_size,
        max_batch=max_batch, swa_window=model.swa_window, swa_period=model.swa_period,
        rope_theta=model.rope_theta, rms_eps=model.rms_eps, expert_fp8=int(model.expert_fp8))


MK_SCHED_UNREACHABLE_WAIT = 1
MK_SCHED_TRACE = 2
MK_SCHED_SEPARATE_TOPK = 4
MK_SCHED_SEPARATE_COMBINE = 8
MK_SCHED_STATIC_MOE = 16
MK_SCHED_SHARED_ATTN = 32
MK_SCHED_SEPARATE_FINALIZE = 64
MK_SCHED_STATIC_ATTN = 128


def make_opts(wave_order="tuned", launch_mode="persistent", attn_split=0, n_workgroups=0,
              timeout_ms=0, flags=0, moe_ug_pairs=0, moe_dn_rows=0) -> mk_sched_opts:
    return mk_sched_opts(wave_order=ORDER[wave_order], launch_mode=LAUNCH[launch_mode],
                         attn_split=attn_split, n_workgroups=n_workgroups, timeout_ms=timeout_ms,
                         flags=flags, moe_ug_pairs=moe_ug_pairs, moe_dn_rows=moe_dn_rows)


def mk_workspace_size(cfg: mk_config, max_blocks_per_seq: int) -> int:
    return int(load().mk_workspace_size(ctypes.byref(cfg), max_blocks_per_seq))


def mk_init(cfg: mk_config, weights: mk_weights, kv: mk_kv_pool, workspace_ptr: int, ws_bytes: int,
            max_blocks_per_seq: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().mk_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv),
                          ctypes.c_void_p(workspace_ptr), ws_bytes, max_blocks_per_seq, ctypes.byref(h)),
           "mk_init")
    return h


def mk_init_noalloc(cfg: mk_config, weights: mk_weights, kv: mk_kv_pool, max_blocks_per_seq: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().mk_init_noalloc(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv), max_blocks_per_seq,
                                  ctypes.byref(h)), "mk_init_noalloc")
    return h


def mk_build_schedule(h, batch_size: int, opts: Optional[mk_sched_opts] = None) -> None:
    _check(load().mk_build_schedule(h, batch_size, ctypes.byref(opts) if opts is not None else None),
           "mk_build_schedule")


def mk_decode_step(h, token_ids: int, positions: int, block_tables: int, seq_lens: int, logits: int,
                   stream: int = 0) -> None:
    _check(load().mk_decode_step(h, ctypes.c_void_p(token_ids), ctypes.c_void_p(positions),
                                 ctypes.c_void_p(block_tables), ctypes.c_void_p(seq_lens),
                                 ctypes.c_void_p(logits), ctypes.c_void_p(stream)), "mk_decode_step")


def mk_decode_step_sample(h, token_ids: int, positions: int, block_tables: int, seq_lens: int, logits: int,
                          sampling: mk_sampling, next_tokens: int, stream: int = 0) -> None:
    _check(load().mk_decode_step_sample(h, ctypes.c_void_p(token_ids), ctypes.c_void_p(positions),
                                        ctypes.c_void_p(block_tables), ctypes.c_void_p(seq_lens),
                                        ctypes.c_void_p(logits), ctypes.byref(sampling),
                                        ctypes.c_void_p(next_tokens), ctypes.c_void_p(stream)),
           "mk_decode_step_sample")


def make_sampling(temperature: float = 0.0, seed: int = 0, advance: bool = False) -> mk_sampling:
    return mk_sampling(temperature=temperature, seed=seed & 0xFFFFFFFF,
                       flags=MK_SAMPLE_ADVANCE if advance else 0)


def mk_get_status(h) -> mk_status:
    st = mk_status()
    load().mk_get_status(h, ctypes.byref(st))
    return st


def mk_tap_offset(h, tap: str) -> tuple:
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().mk_tap_offset(h, TAPS[tap], ctypes.byref(off), ctypes.byref(nb)), "mk_tap_offset")
    return off.value, nb.value


def mk_plan_schedule(cfg: mk_config, batch_size: int, max_blocks_per_seq: int,
                     opts: Optional[mk_sched_opts], n_workgroups: int):
    """Host-only plan: returns (tasks as a list of mk_task, n_counters)."""
    L = load()
    nt, nc = ctypes.c_int32(), ctypes.c_int32()
    o = ctypes.byref(opts) if opts is not None else None
    _check(L.mk_plan_schedule(ctypes.byref(cfg), batch_size, max_blocks_per_seq, o, n_workgroups, None, 0,
                              ctypes.byref(nt), ctypes.byref(nc)), "mk_plan_schedule")
    arr = (mk_task * nt.value)()
    _check(L.mk_plan_schedule(ctypes.byref(cfg), batch_size, max_blocks_per_seq, o, n_workgroups, arr,
                              nt.value, ctypes.byref(nt), ctypes.byref(nc)), "mk_plan_schedule")
    return list(arr), nc.value


def mk_plan_simulate(cfg: mk_config, batch_size: int, max_blocks_per_seq: int,
                     opts: Optional[mk_sched_opts], n_workgroups: int, seq_lens: Sequence[int],
                     n_active_experts: Sequence[int]) -> tuple:
    """Host-only deadlock check: returns (rc, stuck_task)."""
    sl = (ctypes.c_int32 * len(seq_lens))(*seq_lens)
    na = (ctypes.c_int32 * max(1, len(n_active_experts)))(*n_active_experts)
    stuck = ctypes.c_int32(-1)
    o = ctypes.byref(opts) if opts is not None else None
    rc = load().mk_plan_simulate(ctypes.byref(cfg), batch_size, max_blocks_per_seq, o, n_workgroups, sl, na,
                                 ctypes.byref(stuck))
    return rc, stuck.value


def mk_destroy(h) -> None:
    load().mk_destroy(h)
