"""Analysis of the device task trace (schedule flag MK_SCHED_TRACE).

Each task records the 100 MHz device clock when its workgroup reached it,
when its wait was satisfied, and when it finished.  From that:

* per opcode: tasks, total busy time (ready -> end) and total wait time
  (start -> ready) summed over workgroups;
* per layer: when its first task started and its last task ended;
* idle time of each workgroup between its tasks;
* a Chrome trace-event JSON (one row per workgroup) for a timeline viewer.

The wait time splits the bandwidth the pages say a conventional decode loses
(page 4, the four sources of lost bandwidth): time spent waiting on a
producer (false dependencies and the critical path), and time a workgroup
sits idle at the end of the step (the tail a kernel boundary would round up).
"""
from __future__ import annotations

import json
from collections import defaultdict

import numpy as np

from .mk import OPCODES

TICK_US = 0.01   # 100 MHz clock


def load(eng) -> dict:
    """Trace of the last step of a DecodeEngine built with MK_SCHED_TRACE."""
    from . import mk
    tasks, _ = mk.mk_plan_schedule(eng.mkcfg, eng.wl.batch, eng.max_blocks, eng.opts, _n_wg(eng))
    raw = eng.tap("trace").cpu().numpy().reshape(-1, 16)[:len(tasks)]
    return {"tasks": tasks, "raw": raw}


def _n_wg(eng):
    import torch
    if eng.opts.n_workgroups > 0:
        return eng.opts.n_workgroups
    return torch.cuda.get_device_properties(eng.dev).multi_processor_count


def summarize(tr: dict) -> dict:
    tasks, raw = tr["tasks"], tr["raw"].astype(np.int64)
    t0 = raw[:, 0].min()
    start, ready, end, wg = raw[:, 0] - t0, raw[:, 1] - t0, raw[:, 12] - t0, raw[:, 13]
    per_op = defaultdict(lambda: [0, 0.0, 0.0])
    phases = defaultdict(lambda: [[], [], [], []])   # ready->staged, staged->computed, computed->stored, stored->end
    mark_times = defaultdict(lambda: defaultdict(list))   # per opcode: mark -> times after task start
    per_layer = defaultdict(lambda: [np.inf, 0.0])
    for i, t in enumerate(tasks):
        name = OPCODES[t.op]
        s = per_op[name]
        s[0] += 1
        s[1] += (end[i] - ready[i]) * TICK_US
        s[2] += (ready[i] - start[i]) * TICK_US
        # staged (mark 0), the compute waves' last row group (mark 4, set by
        # the first compute wave; mark 1 is the control wave's), stores
        # acknowledged (mark 2)
        st, so = raw[i, 2], raw[i, 4]
        cp = raw[i, 6] if raw[i, 6] >= st and raw[i, 6] else raw[i, 3]
        if st and cp and so:
            ph = phases[name]
            ph[0].append((st - raw[i, 1]) * TICK_US)
            ph[1].append((cp - st) * TICK_US)
            ph[2].append((so - cp) * TICK_US)
            ph[3].append((raw[i, 12] - so) * TICK_US)
        marks = [raw[i, 2 + q] for q in range(10)]
        if any(marks[3:]):
            mm = mark_times[name]
            for q in range(10):
                if marks[q]:
                    mm[q].append((marks[q] - raw[i, 0]) * TICK_US)
            mm["ready"].append((raw[i, 1] - raw[i, 0]) * TICK_US)
            mm["end"].append((raw[i, 12] - raw[i, 0]) * TICK_US)
        pl = per_layer[t.layer]
        pl[0] = min(pl[0], start[i] * TICK_US)
        pl[1] = max(pl[1], end[i] * TICK_US)
    # per-layer critical path: when the last task of each kind in layer l
    # finished (its signal), relative to the end of the norm entering l
    kinds = {"ADD_RMSNORM": "norm", "QKV_PROJ": "qkv", "ROUTER_GEMM": "routing", "ATTN_DRAIN": "attention+combine",
             "ATTN_DECODE": "attention", "ATTN_COMBINE": "combine", "MOE_UPGATE_ACT_DRAIN": "moe_upgate",
             "O_PROJ": "o_proj", "MOE_DOWN_DRAIN": "moe_down", "FFN_UPGATE_ACT": "ffn_upgate", "FFN_DOWN": "ffn_down"}
    last = defaultdict(dict)
    for i, t in enumerate(tasks):
        k = kinds.get(OPCODES[t.op])
        if k is None:
            continue
        e = end[i] * TICK_US
        last[t.layer][k] = max(last[t.layer].get(k, 0.0), e)
    crit = defaultdict(list)
    layers = sorted(l for l in last if "norm" in last[l])
    for l in layers[1:-1]:
        n0 = last[l]["norm"]
        for k, v in last[l].items():
            if k != "norm":
                crit[k].append(v - n0)
        if l + 1 in last and "norm" in last[l + 1]:
            crit["next_norm"].append(last[l + 1]["norm"] - n0)
    step_us = (end.max()) * TICK_US
    n_wg = int(wg.max()) + 1
    idle_tail = float(np.mean([step_us - end[wg == w].max() * TICK_US for w in range(n_wg)]))
    return {
        "step_us": float(step_us),
        "workgroups": n_wg,
        "mean_tail_idle_us": idle_tail,
        "per_op": {k: {"tasks": v[0], "busy_us": round(v[1], 1), "wait_us": round(v[2], 1)}
                   for k, v in sorted(per_op.items(), key=lambda kv: -kv[1][1])},
        "per_layer": {int(k): {"first_start_us": round(v[0], 2), "last_end_us": round(v[1], 2)}
                      for k, v in sorted(per_layer.items())},
        "layer_critical_path_median_us": {k: round(float(np.median(v)), 2)
                                          for k, v in sorted(crit.items(), key=lambda kv: np.median(kv[1]))},
        "phases_median_us": {k: {"stage": round(float(np.median(v[0])), 2),
                                 "compute": round(float(np.median(v[1])), 2),
                                 "store_ack": round(float(np.median(v[2])), 2),
                                 "tail": round(float(np.median(v[3])), 2)}
                             for k, v in phases.items() if v[0]},
        "marks_median_us_from_start": {k: {str(q): round(float(np.median(v)), 2) for q, v in sorted(m.items(), key=str)}
                                       for k, m in mark_times.items()},
    }


def chrome_trace(tr: dict, path: str) -> None:
    tasks, raw = tr["tasks"], tr["raw"].astype(np.int64)
    t0 = raw[:, 0].min()
    ev = []
    for i, t in enumerate(tasks):
        s, r, e, w = (raw[i, 0] - t0) * TICK_US, (raw[i, 1] - t0) * TICK_US, (raw[i, 12] - t0) * TICK_US, raw[i, 13]
        name = f"{OPCODES[t.op]} L{t.layer}"
        if r > s:
            ev.append({"name": "wait " + name, "ph": "X", "ts": float(s), "dur": float(r - s), "pid": 0,
                       "tid": int(w), "cat": "wait"})
        ev.append({"name": name, "ph": "X", "ts": float(r), "dur": float(max(e - r, 0)), "pid": 0,
                   "tid": int(w), "cat": OPCODES[t.op]})
    with open(path, "w") as fh:
        json.dump({"traceEvents": ev}, fh)
