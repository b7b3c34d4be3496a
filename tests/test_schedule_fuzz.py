"""Seeded random schedules through the host deadlock simulator (no GPU).

Every wave order and schedule flag, on grids of 4 to 256 workgroups, for
batches of 1 to 8 with ragged and empty slots, short and long contexts
(including contexts whose splits make the tuned order use attention owners)
and any number of distinct routed experts: the planned task lists must drain
(mk_plan_simulate returns MK_OK)."""
import random
from dataclasses import replace

import pytest

from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W

# the real head and expert geometry with few layers (the schedule of a layer
# does not depend on the others), and the sliding-window variant
MOE_3L = replace(W.MOE_30B, name="moe30b-shape-3l", n_layers=3)
SWA_4L = replace(W.MOE_30B_SWA, name="moe30b-swa-4l", n_layers=4)
DENSE_2L = replace(W.DENSE_1B, name="dense1b-shape-2l", n_layers=2)
MODELS = [W.TINY_MOE, MOE_3L, SWA_4L, DENSE_2L]

ORDERS = ["tuned", "interleaved", "attention_first", "partitioned"]
FLAGS = [0, mk.MK_SCHED_SEPARATE_TOPK, mk.MK_SCHED_SEPARATE_TOPK | mk.MK_SCHED_SEPARATE_FINALIZE,
         mk.MK_SCHED_SEPARATE_COMBINE, mk.MK_SCHED_STATIC_MOE, mk.MK_SCHED_STATIC_ATTN, mk.MK_SCHED_SHARED_ATTN]


@pytest.fixture(scope="module")
def lib():
    return mk.load()


def _case(rng: random.Random):
    model = rng.choice(MODELS)
    # the dense model stages B rows of its 8192-wide FFN input: at most 2
    B = rng.randint(1, 8 if model.n_experts else 2)
    nw = rng.choice([4, 7, 16, 40, 64, 128, 200, 250, 256])
    page = 16
    # longest context: short, around the owner range at bs=1 (a few
    # thousand keys), or long
    max_ctx = rng.choice([page * rng.randint(1, 8), rng.randint(1000, 12000), rng.randint(12000, 40000)])
    mb = -(-max_ctx // page)
    sl = [0 if (b > 0 and rng.random() < 0.2) else rng.randint(1, mb * page) for b in range(B)]
    if model.n_experts:
        cap = min(model.n_experts, B * model.top_k)
        na = [rng.randint(1, cap) for _ in range(model.n_layers)]
    else:
        na = []
    order = rng.choice(ORDERS)
    flags = rng.choice(FLAGS)
    return model, B, nw, mb, sl, na, order, flags


def _planned(model, B, nw, mb, order, flags):
    """False when the builder refuses the shape up front (for example a QKV
    tile of the 30B shape on 4 workgroups is larger than its LDS output)."""
    try:
        mk.mk_plan_schedule(mk.make_config(model, B), B, mb, mk.make_opts(order, flags=flags), nw)
    except RuntimeError as e:
        assert "unsupported" in str(e), e
        return False
    return True


@pytest.mark.parametrize("seed", range(200))
def test_random_schedule_drains(lib, seed):
    rng = random.Random(1000 + seed)
    model, B, nw, mb, sl, na, order, flags = _case(rng)
    opts = mk.make_opts(order, flags=flags)
    cfg = mk.make_config(model, B)
    rc, stuck = mk.mk_plan_simulate(cfg, B, mb, opts, nw, sl, na)
    if not _planned(model, B, nw, mb, order, flags):
        assert rc == mk.MK_E_UNSUPPORTED
        return
    assert rc == mk.MK_OK, (model.name, B, nw, mb, sl, na, order, flags, stuck)


def test_random_cases_are_mostly_plannable(lib):
    n = sum(_planned(*(lambda c: (c[0], c[1], c[2], c[3], c[6], c[7]))(_case(random.Random(1000 + s))))
            for s in range(200))
    assert n >= 150, n


def _owner_case(rng: random.Random):
    """Tuned order at one or two rows with contexts of a few thousand keys,
    where the splits number between a quarter and half of the grid."""
    model = rng.choice([MOE_3L, SWA_4L])
    B = rng.randint(1, 2)
    nw = rng.choice([64, 128, 200, 256])
    mb = -(-rng.randint(1500, 12000) // 16)
    sl = [rng.randint(1, mb * 16) for _ in range(B)]
    na = [rng.randint(1, B * model.top_k) for _ in range(model.n_layers)]
    flags = rng.choice([0, mk.MK_SCHED_STATIC_MOE])
    return model, B, nw, mb, sl, na, flags


@pytest.mark.parametrize("seed", range(100))
def test_random_owner_schedule_drains(lib, seed):
    model, B, nw, mb, sl, na, flags = _owner_case(random.Random(5000 + seed))
    rc, stuck = mk.mk_plan_simulate(mk.make_config(model, B), B, mb, mk.make_opts("tuned", flags=flags), nw, sl, na)
    assert rc == mk.MK_OK, (model.name, B, nw, mb, sl, na, flags, stuck)


def test_random_owner_cases_reach_the_owner_schedule(lib):
    owners = 0
    for seed in range(100):
        model, B, nw, mb, sl, na, flags = _owner_case(random.Random(5000 + seed))
        tasks, _ = mk.mk_plan_schedule(mk.make_config(model, B), B, mb, mk.make_opts("tuned", flags=flags), nw)
        n = sum(1 for t in tasks if t.layer == model.n_layers - 1 and mk.OPCODES[t.op] == "ATTN_DRAIN")
        owners += 0 < n < nw
    assert owners >= 40, owners
