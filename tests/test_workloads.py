"""The seeded input generator and the workload plans (host only)."""
import math

import numpy as np
import pytest
import torch

from persistent_moe_amd import workloads as W


def test_fmix32_reference_values():
    # MurmurHash3 fmix32 of 0 is 0 and of 1 is 0x514E28B7.
    assert W.fmix32_int(0) == 0
    assert W.fmix32_int(1) == 0x514E28B7
    t = W._fmix32(torch.tensor([0, 1, 2 ** 32 - 1]), W._TorchOps("cpu")).tolist()
    n = W._fmix32(np.array([0, 1, 2 ** 32 - 1], dtype=np.uint64), W._NumpyOps).tolist()
    assert t == n == [0, 0x514E28B7, W.fmix32_int(2 ** 32 - 1)]


@pytest.mark.parametrize("start,count", [(0, 5000), (2 ** 32 - 2500, 5000), (3 << 33, 4096)])
def test_backends_bit_identical(start, count):
    a = W.normal_bf16(77, start, count, 0.0, 0.02, backend="numpy").view(torch.int16)
    t = W.normal_bf16(77, start, count, 0.0, 0.02, backend="torch").view(torch.int16)
    assert torch.equal(a, t)
    if W._host_lib() is not None:
        c = W.normal_bf16(77, start, count, 0.0, 0.02, backend="c").view(torch.int16)
        assert torch.equal(a, c)


def test_transform_matches_library_log_and_cos():
    h1, h2 = W._words(9, 0, 1 << 16, W._NumpyOps)
    a = W._neg2_ln_u(h1, W._NumpyOps)
    b = -2 * np.log((h1.astype(np.float64) + 0.5) / 2 ** 32)
    assert np.max(np.abs(a - b) / np.abs(b)) < 4e-15
    a = W._cos_2pi_u(h2, W._NumpyOps)
    b = np.cos(2 * np.pi * (h2.astype(np.float64) + 0.5) / 2 ** 32)
    assert np.max(np.abs(a - b)) < 4e-15


def test_normal_moments():
    x = W.normal_bf16(5, 0, 1 << 20, 0.0, 1.0).double()
    assert abs(x.mean().item()) < 5e-3
    assert abs(x.std().item() - 1) < 5e-3
    tail = (x.abs() > 3).double().mean().item()
    assert abs(tail - 2 * (1 - 0.5 * (1 + math.erf(3 / math.sqrt(2))))) < 5e-4
    g = W.normal_bf16(6, 0, 1 << 16, 1.0, 0.1).double()
    assert abs(g.mean().item() - 1) < 2e-3 and abs(g.std().item() - 0.1) < 2e-3


def test_row_slice_equals_slice_of_whole_tensor():
    full = W.gen_tensor(3, "w_qkv", (40, 24), layer=1)
    part = W.gen_tensor(3, "w_qkv", (40, 24), layer=1, rows=slice(17, 29))
    assert torch.equal(full[17:29].view(torch.int16), part.view(torch.int16))


def test_streams_differ_by_name_layer_expert_seed():
    keys = {W.tensor_key(0, "w_o", 0), W.tensor_key(0, "w_o", 1), W.tensor_key(0, "w_qkv", 0),
            W.tensor_key(1, "w_o", 0), W.tensor_key(0, "w_down", 0, 3), W.tensor_key(0, "w_down", 0, 4)}
    assert len(keys) == 6


def test_kv_slice_equals_slice_of_whole():
    cfg = W.TINY_MOE
    full = W.gen_kv(0, cfg, 2, 1, "k", 0, 50)
    part = W.gen_kv(0, cfg, 2, 1, "k", 13, 37)
    assert torch.equal(full[13:37].view(torch.int16), part.view(torch.int16))


def test_batch_plan_pages_unique_and_sufficient():
    wl = W.WORKLOADS["moe30b_bs8"]
    plan = W.plan_batch(wl)
    pages = W.page_table(plan)
    allp = np.concatenate(list(pages.values()))
    assert len(np.unique(allp)) == len(allp) and allp.max() < plan.num_pages
    for b in range(wl.batch):
        segs = plan.slots[b]
        for i, (first, seq) in enumerate(segs):
            last = segs[i + 1][0] if i + 1 < len(segs) else wl.steps
            assert len(pages[seq.seq_id]) * 16 >= seq.ctx + (last - first)
            assert 512 <= seq.ctx <= 16384
    # one sequence swapped every 32 steps
    assert sum(len(s) - 1 for s in plan.slots) == len(range(32, wl.steps, 32))


def test_start_tokens_in_vocab_and_seeded():
    a = [W.start_token(0, i, 1024) for i in range(50)]
    assert a == [W.start_token(0, i, 1024) for i in range(50)]
    assert all(0 <= t < 1024 for t in a) and len(set(a)) > 30


def test_keyed_vectorised_generator_matches_per_stream():
    keys = [W.tensor_key(2, "w_down", 5, e) for e in range(5)]
    ref = torch.stack([W.gen_tensor(2, "w_down", (40, 24), layer=5, expert=e) for e in range(5)])
    for ge in (1 << 25, 500, 2000):
        out = torch.empty(5, 40, 24, dtype=torch.bfloat16)
        W.fill_normal_keyed_(out, keys, 0.0, 0.02, group_elems=ge, backend="torch")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
