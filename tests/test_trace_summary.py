"""The device task-trace summary (persistent_moe_amd.trace.summarize) on a
synthetic trace whose answers are known: per-opcode busy and wait sums, the
per-layer critical path relative to the norm entering each layer, and the
idle tail of each workgroup."""
import numpy as np

from persistent_moe_amd import mk
from persistent_moe_amd import trace as T

OP = {n: i for i, n in enumerate(mk.OPCODES)}


def _trace(rows):
    """rows: (opcode name, layer, workgroup, start, ready, end) in clock ticks."""
    tasks, raw = [], np.zeros((len(rows), 16), dtype=np.int64)
    for i, (name, layer, wg, start, ready, end) in enumerate(rows):
        t = mk.mk_task()
        t.op, t.layer = OP[name], layer
        tasks.append(t)
        raw[i, 0], raw[i, 1], raw[i, 12], raw[i, 13] = start, ready, end, wg
    return {"tasks": tasks, "raw": raw}


def test_summary_of_a_known_trace():
    # three layers on two workgroups; per layer (ticks of 10 ns) the norm ends
    # at 100 L, QKV ends 300 later, the up-gate drain 700 later, the down drain
    # 1000 later; layer 1's numbers are the only ones of the middle layers
    rows = []
    for l in range(3):
        base = 100 + 1500 * l
        rows += [("ADD_RMSNORM", l, 0, base - 100, base - 50, base),
                 ("QKV_PROJ", l, 0, base, base + 100, base + 300),
                 ("QKV_PROJ", l, 1, base, base + 50, base + 250),
                 ("MOE_UPGATE_ACT_DRAIN", l, 1, base + 300, base + 320, base + 700),
                 ("MOE_DOWN_DRAIN", l, 0, base + 700, base + 710, base + 1000)]
    rows.append(("ADD_RMSNORM", 3, 0, 4600 - 100, 4600 - 50, 4600))
    s = T.summarize(_trace(rows))
    cp = s["layer_critical_path_median_us"]
    # median over the layers between the first and the last (layer 1 and 2)
    assert cp["qkv"] == 3.0 and cp["moe_upgate"] == 7.0 and cp["moe_down"] == 10.0
    assert cp["next_norm"] == 15.0
    po = s["per_op"]
    assert po["QKV_PROJ"]["tasks"] == 6
    assert abs(po["QKV_PROJ"]["busy_us"] - 3 * (2.0 + 2.0)) < 1e-9
    assert abs(po["QKV_PROJ"]["wait_us"] - 3 * (1.0 + 0.5)) < 1e-9
    assert abs(po["MOE_DOWN_DRAIN"]["busy_us"] - 3 * 2.9) < 1e-9
    assert s["workgroups"] == 2
    # the step ends with the last norm (4600 ticks after the first start at 0);
    # workgroup 1 finished its last task at 3100 + 700 = 3800
    assert abs(s["step_us"] - 46.0) < 1e-9
    assert abs(s["mean_tail_idle_us"] - (0.0 + (4600 - 3800) * 0.01) / 2) < 1e-9
