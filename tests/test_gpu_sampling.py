"""The next token picked on the device after LM_HEAD (mk_decode_step_sample),
against the oracle's sampler applied to the same step's logits.

Greedy is an argmax over the fp32 logits the step returns, so it is compared
bit for bit (ties to the lowest id).  Temperature sampling adds Gumbel noise
computed in single precision on the device and in double precision in the
oracle: a decision whose two best perturbed scores lie closer than 1e-3 may go
either way (a near tie), any other must be identical.
"""
import numpy as np
import pytest
import torch

from oracle import decode as O
from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W
from tests.parity import say

pytestmark = pytest.mark.gpu
NEAR_TIE = 1e-3

MOE_SMALL = W.ModelConfig(name="moe30b-shape-2l", n_layers=2, d_model=2048, n_q_heads=32, n_kv_heads=4,
                          head_dim=128, vocab=4096, n_experts=128, top_k=8, expert_inter=768)


@pytest.fixture(scope="module", autouse=True)
def _gpu(gpu_available):
    mk.load()
    yield


def _engine(wl, **kw):
    from persistent_moe_amd.runner import DecodeEngine
    say("engine", wl.name, "B", wl.batch, kw)
    return DecodeEngine(wl, **kw)


def _step(eng, smp, inputs=None):
    t, pos, sl = inputs if inputs is not None else eng.step_inputs()
    nxt = torch.full((eng.wl.batch,), -7, dtype=torch.int32, device=eng.dev)
    s = torch.cuda.current_stream()
    mk.mk_decode_step_sample(eng.h, t.data_ptr(), pos.data_ptr(), eng.block_tables.data_ptr(), sl.data_ptr(),
                             eng.logits.data_ptr(), smp, nxt.data_ptr(), s.cuda_stream)
    st = eng.status()
    assert st.code == 0, st.code
    return nxt.cpu().numpy(), eng.logits.cpu().numpy(), (t, pos, sl)


@pytest.mark.parametrize("wl,kw", [
    (W.Workload("tiny-bs4-sample", W.TINY_MOE, batch=4, ctx="list:40,64,9,100", steps=1, seed=31), {}),
    (W.Workload("moe30b-shape-sample", MOE_SMALL, batch=2, ctx="list:300,77", steps=1, seed=32), {}),
    (W.Workload("moe30b-shape-sample-12wg", MOE_SMALL, batch=2, ctx="list:300,77", steps=1, seed=33),
     {"opts": mk.make_opts(n_workgroups=12)}),
], ids=["tiny-bs4", "moe30b-shape-256-tiles", "moe30b-shape-12wg"])
def test_greedy_next_token_is_argmax_of_the_logits(wl, kw):
    eng = _engine(wl, **kw)
    t, pos, sl = eng.step_inputs()
    if wl.batch == 4:
        sl[2] = 0                                   # an empty slot gets -1
    nxt, lg, _ = _step(eng, mk.make_sampling(0.0), (t, pos, sl))
    for b in range(wl.batch):
        want = -1 if (wl.batch == 4 and b == 2) else int(np.argmax(lg[b]))
        assert nxt[b] == want, (b, nxt, want)
    # the logits equal those of the plain step
    ref = eng.decode(inputs=(t, pos, sl)).cpu().numpy()
    assert np.array_equal(ref, lg)


@pytest.mark.parametrize("T,seed", [(0.7, 5), (1.0, 123), (2.5, 77)])
def test_temperature_sample_matches_oracle_sampler(T, seed):
    wl = W.Workload("moe30b-shape-temp", MOE_SMALL, batch=2, ctx="list:200,31", steps=64, seed=34)
    eng = _engine(wl)          # pages for 64 more positions: the draws below move ahead 48
    decided = 0
    inp = eng.step_inputs()
    for rep in range(4):
        t, pos, sl = inp
        pos2, sl2 = pos + 16 * rep, sl + 16 * rep  # other positions draw other noise
        nxt, lg, _ = _step(eng, mk.make_sampling(T, seed), (t, pos2, sl2))
        for b in range(wl.batch):
            tok, gap = O.sample_token(lg[b].astype(np.float64), T, seed, int(pos2[b]), b)
            if gap >= NEAR_TIE:
                assert nxt[b] == tok, (rep, b, nxt[b], tok, gap)
                decided += 1
            else:
                z = lg[b].astype(np.float64) / T - np.log(-np.log(O.sampling_uniforms(seed, int(pos2[b]), b, wl.model.vocab)))
                assert nxt[b] in np.argsort(z)[-2:]
    assert decided >= 6
    say(f"temperature {T}: {decided} decided draws equal")


def test_advance_runs_steps_back_to_back_like_the_oracle_greedy_decode():
    """Six steps enqueued with no host work between them (the kernel feeds the
    sampled token back and advances positions and lengths), against the
    oracle's greedy decode of the same seeded start."""
    wl = W.WORKLOADS["tiny"].with_(batch=2, ctx="list:64,20")
    steps = 6
    eng = _engine(wl, steps=steps)
    t, pos, sl = eng.step_inputs()
    pos0 = pos.cpu().numpy().copy()
    outs = [torch.full((2,), -7, dtype=torch.int32, device=eng.dev) for _ in range(steps)]
    logs = []
    s = torch.cuda.current_stream()
    smp = mk.make_sampling(0.0, advance=True)
    for i in range(steps):
        mk.mk_decode_step_sample(eng.h, t.data_ptr(), pos.data_ptr(), eng.block_tables.data_ptr(), sl.data_ptr(),
                                 eng.logits.data_ptr(), smp, outs[i].data_ptr(), s.cuda_stream)
        logs.append(eng.logits.clone())
    assert eng.status().code == 0
    assert np.array_equal(pos.cpu().numpy(), pos0 + steps)
    assert np.array_equal(sl.cpu().numpy(), pos0 + steps + 1)
    toks = np.stack([o.cpu().numpy() for o in outs])     # [steps][B]
    assert np.array_equal(t.cpu().numpy(), toks[-1])
    fed, res = O.greedy_decode(wl, steps)
    compared = 0
    for b in range(2):
        for i in range(steps):
            r = res[i][b]
            err = float(np.max(np.abs(logs[i][b].cpu().numpy() - r.logits)))
            assert err <= 2e-2 * float(np.std(r.logits)), (i, b, err)
            compared += 1
            top2 = np.sort(r.logits)[-2:]
            if top2[1] - top2[0] < 1e-3 * np.std(r.logits):
                # a near tie may go either way; the slot's later steps then
                # follow another history, so they are not compared
                assert toks[i, b] in np.argsort(r.logits)[-2:]
                break
            assert toks[i, b] == r.token, (i, b)
    assert compared >= steps
