"""mk_init_noalloc: a handle whose workspace is the library's per-device
scratch array instead of a caller allocation.  Its steps are checked against
those of mk_init (caller workspace) on the same weights, KV pools and inputs,
bit for bit, on two calls in a row, the second with a smaller input; and a
model whose workspace exceeds the array is refused."""
import ctypes

import pytest
import torch

from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W

pytestmark = pytest.mark.gpu

MOE_SMALL = W.ModelConfig(name="moe30b-shape-2l", n_layers=2, d_model=2048, n_q_heads=32, n_kv_heads=4,
                          head_dim=128, vocab=4096, n_experts=128, top_k=8, expert_inter=768)


def _say(*a):
    print("[no-alloc]", *a, flush=True)


def test_noalloc_handle_matches_caller_workspace(gpu_available):
    from persistent_moe_amd.runner import DecodeEngine
    mk.load()
    cases = [
        W.Workload("moe30b-shape-noalloc", MOE_SMALL, batch=2, ctx="list:8192,3000", steps=2, seed=41),
        W.Workload("tiny-noalloc", W.TINY_MOE, batch=1, ctx="list:20", steps=2, seed=42),   # smaller
    ]
    for wl in cases:
        _say("case", wl.name)
        eng = DecodeEngine(wl)              # mk_init with a caller workspace
        inp = eng.step_inputs()
        ref = eng.decode(inputs=inp).clone()
        assert eng.status().code == 0
        h = mk.mk_init_noalloc(eng.mkcfg, eng._w, eng._kv, eng.max_blocks)
        mk.mk_build_schedule(h, wl.batch, mk.make_opts())
        out = torch.full_like(eng.logits, float("nan"))
        t, pos, sl = inp
        mk.mk_decode_step(h, t.data_ptr(), pos.data_ptr(), eng.block_tables.data_ptr(), sl.data_ptr(),
                          out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert mk.mk_get_status(h).code == 0
        assert torch.equal(out, ref), float((out - ref).abs().max())
        # the handle uses no trace region
        with pytest.raises(mk.MkError):
            mk.mk_build_schedule(h, wl.batch, mk.make_opts(flags=mk.MK_SCHED_TRACE))
        mk.mk_destroy(h)
        eng.close()
        torch.cuda.synchronize()


def test_noalloc_refuses_a_workspace_larger_than_the_array(gpu_available):
    mk.load()
    cfg = mk.make_config(W.MOE_30B, 8)
    L = cfg.n_layers
    # placeholder pointers: the size check fails before anything is read
    arr = (mk.mk_layer_weights * L)()
    for l in range(L):
        for f in ("attn_norm", "w_qkv", "w_o", "w_router", "w_upgate", "w_down"):
            setattr(arr[l], f, 256)
    w = mk.mk_weights(embed=256, lm_head=256, final_norm=256, layers=arr)
    kp = (ctypes.c_void_p * L)(*([256] * L))
    kv = mk.mk_kv_pool(k=kp, v=kp, num_pages=100000)
    h = ctypes.c_void_p()
    rc = mk.load().mk_init_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), 1026, ctypes.byref(h))
    assert rc == mk.MK_E_NOMEM and not h.value
