"""Decode throughput of the persistent decode megakernel on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload moe30b]

Times K greedy decode steps (after W untimed ones) of the 30B / 3.3B-active
parallel-block MoE at batch 1 with an 8K-token pre-filled paged KV cache,
random-init bf16 weights from the seeded generator.  Each step is one
mk_decode_step_sample launch: the whole decode step in one persistent kernel,
with the greedy next token picked on the device after LM_HEAD and the slots
advanced by the kernel, so the timed loop launches nothing else and never
synchronises with the host.  Prints one JSON line, which also carries the
batch-8 leg of the metric (the ragged continuous-batching workload) and the
wave-order / one-launch-per-wave ablation.

Reported next to the throughput:
* roofline: speed-of-light bytes of every step (active weights read once, KV
  of every visible key), over the kernel's own average duration measured with
  events on its stream, against the 8 TB/s HBM peak;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at bs1 and bs8; % of HBM speed-of-light, 30B/3.3B-active MoE"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["persistent_moe_amd/csrc/mk_kernel.hip", "persistent_moe_amd/csrc/mk_host.cpp",
                  "persistent_moe_amd/csrc/mk_internal.h"]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken with the kernel sources as they are now and for this workload; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "mk_persistent_moe30b_bs1_ctx8k_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if kv.get("kernel_sources_sha256_16") != h.hexdigest()[:16] or kv.get("workload") != workload:
        return None
    return int(kv["fetch_bytes"]) + int(kv["write_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="moe30b")
    ap.add_argument("--order", default="tuned")
    ap.add_argument("--launch", default="persistent")
    ap.add_argument("--attn-split", type=int, default=0)
    ap.add_argument("--sched-flags", type=int, default=0, help="MK_SCHED_* bits for the schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bs8", action="store_true", help="skip the batch-8 leg of the metric")
    ap.add_argument("--no-ablation", action="store_true", help="skip the wave-order / per-opcode ablation")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-expert leg")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--trace", default="", help="after timing, trace one step and write a summary here")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the steps, run an elementwise kernel that reads and writes this many MiB "
                         "(3 times): known traffic to scale HBM byte counters by")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(wl, sample_layers: int = 4, lm_frac: int = 16, min_seconds: float = 10.0):
    """Time the CPU oracle on a bounded sample of one decode step.

    The sample is the first ``sample_layers`` layers of the same seeded model
    plus 1/``lm_frac`` of its LM-head rows; a layerless run of the same
    sample isolates the LM-head time.  Weight and cache generation happen
    before the timed runs.  Scaled to a full step:
    t = (t_sample - t_head) / sample_layers * n_layers + t_head * lm_frac.
    """
    from oracle import decode as O
    from persistent_moe_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cfg = wl.model
    V = cfg.vocab // lm_frac
    swl = wl.with_(model=replace(cfg, n_layers=sample_layers, vocab=V))
    hwl = wl.with_(model=replace(cfg, n_layers=0, vocab=V))
    plan = W.plan_batch(swl, 1)
    seqs0 = [plan.slots[b][0][1] for b in range(wl.batch)]

    def run(w, Wt, keep):
        seqs = [O.new_sequence(s.seq_id, s.ctx) for s in seqs0]
        for s, k in zip(seqs, keep):
            s.prefill_cache = k
        t0 = time.perf_counter()
        O.decode_step(w, Wt, seqs, [s.token for s in seqs0])
        return time.perf_counter() - t0, [s.prefill_cache for s in seqs]

    Ws = O.Weights(swl, cache_limit=64 << 30)
    Wh = O.Weights(hwl, cache_limit=64 << 30)
    for w in (Ws, Wh):     # draw the LM-head sample rows once, outside the timing
        w.lm_head_rows = (lambda f: (lambda r0, r1, _c={}: _c.setdefault((r0, r1), f(r0, r1))))(w.lm_head_rows)
    _, keep = run(swl, Ws, [{}] * wl.batch)          # warm: generate weights and cache
    run(hwl, Wh, keep)
    reps, ts, th = 0, [], []
    t_begin = time.perf_counter()
    while True:
        a, _ = run(swl, Ws, keep)
        b, _ = run(hwl, Wh, keep)
        ts.append(a)
        th.append(b)
        reps += 1
        if time.perf_counter() - t_begin >= min_seconds or reps >= 50:
            break
    t_s, t_h = float(np.median(ts)), float(np.median(th))
    t_layer = max(t_s - t_h, 0.0) / sample_layers
    t_step = t_layer * cfg.n_layers + t_h * lm_frac
    return {
        "value": wl.batch / t_step,
        "unit": "tok/s",
        "cores": threads,
        "kind": "oracle",
        "ms_per_step": t_step * 1e3,
        "sample": (f"{sample_layers} of {cfg.n_layers} layers and 1/{lm_frac} of the LM-head rows of "
                   f"step 0 (fp64 numpy, weights drawn before timing), median of {reps} runs, "
                   f"scaled to a full step"),
    }


def time_steps(eng, n_warm: int, n_steps: int, route_log_every: bool = True):
    """Warm up, then time n_steps decode steps enqueued back to back.

    Each step is one mk_decode_step_sample launch with greedy sampling and
    MK_SAMPLE_ADVANCE: the kernel picks the next token after LM_HEAD and
    advances the slots' tokens, positions and lengths itself, so the loop
    runs no other kernel and needs no host synchronisation.  Returns the
    wall time of the timed steps, the per-launch event times (ms) on the
    launch stream, the positions before the first timed step and the routed
    expert ids of every timed step (batch > 1), for the exact byte count.
    """
    import torch

    from persistent_moe_amd import mk

    wl, cfg, B = eng.wl, eng.cfg, eng.wl.batch
    stream = torch.cuda.current_stream()
    tok, pos, sl = eng.step_inputs()
    nxt = torch.zeros(B, dtype=torch.int32, device=eng.dev)
    smp = mk.make_sampling(0.0, advance=True)
    ids_tap = eng.tap("topk_ids") if cfg.is_moe else None
    L, K = cfg.n_layers, max(cfg.top_k, 1)
    route_log = (torch.zeros((n_steps, L * B * K), dtype=torch.int32, device=eng.dev)
                 if cfg.is_moe and B > 1 and route_log_every else None)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]

    def launch():
        mk.mk_decode_step_sample(eng.h, tok.data_ptr(), pos.data_ptr(), eng.block_tables.data_ptr(),
                                 sl.data_ptr(), eng.logits.data_ptr(), smp, nxt.data_ptr(), stream.cuda_stream)

    for _ in range(n_warm):
        launch()
    torch.cuda.synchronize()
    st = eng.status()
    if st.code != 0:
        raise SystemExit(f"device error during warmup: {mk.strerror(st.code)} task {st.task}")
    pos0 = pos.cpu().numpy().copy()
    t0 = time.perf_counter()
    for i in range(n_steps):
        ev[i][0].record(stream)
        launch()
        ev[i][1].record(stream)
        if route_log is not None:
            route_log[i].copy_(ids_tap[:L * B * K])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = eng.status()
    if st.code != 0:
        raise SystemExit(f"device error: {mk.strerror(st.code)} task {st.task} counter {st.counter}")
    eng.slot_len = [int(v) for v in sl.cpu().numpy() - 1]   # the kernel advanced the slots
    eng.slot_tok = [int(v) for v in tok.cpu().numpy()]
    kern = [a.elapsed_time(b) for a, b in ev]
    return wall, kern, pos0, (route_log.cpu().numpy() if route_log is not None else None)


def step_metrics(cfg, B, wall, kern, pos0, rl, n_steps):
    """tok/s, ms/step and the kernel's roofline from the exact bytes of every
    timed step (active weights read once + the KV of every visible key)."""
    from persistent_moe_amd import sol

    L, K = cfg.n_layers, max(cfg.top_k, 1)
    step_bytes = []
    for i in range(n_steps):
        p = (pos0 + i).tolist()
        if rl is not None:
            ids = rl[i].reshape(L, B, K)
            distinct = [len(np.unique(ids[l])) for l in range(L)]
        else:
            distinct = [K if cfg.is_moe else 0] * L
        step_bytes.append(sol.step_bytes(cfg, p, distinct))
    mean_bytes = float(np.mean(step_bytes))
    mean_kern_s = float(np.mean(kern)) / 1e3
    achieved = mean_bytes / mean_kern_s / 1e9
    sol_tok_s = float(np.mean([sol.sol_tok_s(b, B) for b in step_bytes]))
    value = B * n_steps / wall
    return {
        "value": round(value, 2),
        "ms_per_step": round(wall / n_steps * 1e3, 4),
        "kernel_ms": round(mean_kern_s * 1e3, 4),
        "sol_tok_s": round(sol_tok_s, 1),
        "sol_fraction": round(value / sol_tok_s, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_step": int(mean_bytes), "kernel": "mk_persistent"},
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the decode step runs in one persistent kernel on one device).", file=sys.stderr)
        sys.exit(2)
    import torch

    from persistent_moe_amd import mk
    from persistent_moe_amd import workloads as W
    from persistent_moe_amd.runner import DecodeEngine

    wl = W.WORKLOADS[args.workload]
    cfg = wl.model
    B = wl.batch
    abl_steps = 0 if args.no_ablation else 16
    ablation = [("interleaved", "persistent"), ("attention_first", "persistent"), ("tuned", "per_opcode")]
    total_steps = args.warmup + args.steps + len(ablation) * (abl_steps + 2)
    log(f"workload {wl.name}: building inputs for {total_steps} steps")
    t0 = time.time()
    opts = mk.make_opts(args.order, args.launch, attn_split=args.attn_split, flags=args.sched_flags)
    eng = DecodeEngine(wl, steps=total_steps + 1, opts=opts, verbose=args.verbose)
    log(f"inputs ready in {time.time() - t0:.1f}s ({eng.weight_bytes() / 1e9:.1f} GB weights)")
    if wl.swap_every:
        log("note: slot swaps are not applied inside the timed loop")
    if args.calib_copy_mib:
        # an elementwise kernel (negation) that reads and writes exactly n bytes
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration kernel: 3 x ({args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written)")
        del src, dst
    wall, kern, pos0, rl = time_steps(eng, args.warmup, args.steps)
    m = step_metrics(cfg, B, wall, kern, pos0, rl, args.steps)
    m["roofline"]["traffic"] = measured_traffic(wl.name)
    log(f"{m['value']:.1f} tok/s, {m['ms_per_step']:.3f} ms/step; kernel {m['kernel_ms']:.3f} ms "
        f"(min {min(kern):.3f}); {m['roofline']['achieved']:.0f} GB/s = {m['roofline']['frac']:.1%} of HBM SoL")
    out = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and pre-filled KV)",
        "config": {"workload": wl.name, "batch": B, "context": W.context_length(wl, 0),
                   "layers": cfg.n_layers, "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "order": args.order, "launch": args.launch, "sched_flags": args.sched_flags,
                   "attn_split": args.attn_split or "auto", "sampling": "greedy, on device, fused after LM_HEAD"},
        "sol_fraction": m["sol_fraction"],
        "sol_tok_s": m["sol_tok_s"],
        "kernel_ms": m["kernel_ms"],
        "roofline": m["roofline"],
    }
    if abl_steps:
        # the pages' scheduling ablation (tuned vs interleaved vs attention-first
        # wave orders) and one launch per task wave instead of the megakernel,
        # on the same engine and inputs
        abl = {"tuned": {"tok_s": m["value"], "kernel_ms": m["kernel_ms"]}}
        for order, launch in ablation:
            mk.mk_build_schedule(eng.h, B, mk.make_opts(order, launch))
            w2, k2, _, _ = time_steps(eng, 2, abl_steps, route_log_every=False)
            name = order if launch == "persistent" else "per_opcode_launch"
            abl[name] = {"tok_s": round(B * abl_steps / w2, 2), "kernel_ms": round(float(np.mean(k2)), 4)}
            log(f"ablation {name}: {abl[name]['tok_s']:.1f} tok/s")
        mk.mk_build_schedule(eng.h, B, opts)
        out["ablation"] = abl
    if args.trace:
        from persistent_moe_amd import trace as T
        topt = mk.make_opts(args.order, args.launch, attn_split=args.attn_split,
                            flags=args.sched_flags | mk.MK_SCHED_TRACE)
        eng.opts = topt
        mk.mk_build_schedule(eng.h, B, topt)
        time_steps(eng, 0, 1, route_log_every=False)
        tr = T.load(eng)
        summ = T.summarize(tr)
        with open(args.trace, "w") as fh:
            json.dump(summ, fh, indent=1)
        T.chrome_trace(tr, os.path.splitext(args.trace)[0] + ".chrome.json")
        log(f"trace: step {summ['step_us']:.1f} us; " +
            ", ".join(f"{k} busy {v['busy_us']:.0f} wait {v['wait_us']:.0f}" for k, v in summ["per_op"].items()))
    # release this engine before the batch-8 leg (explicit teardown: every
    # launch has completed before the handle and the buffers go)
    torch.cuda.synchronize()
    eng.close()
    del eng
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    legs = []
    if not args.no_bs8 and args.workload == "moe30b":
        # the batch-8 leg of the metric: uniform routing (random router) and
        # concentrated routing (Zipf router bias), ragged contexts
        legs += [("bs8", "moe30b_bs8"), ("bs8_zipf", "moe30b_bs8_zipf")]
    if not args.no_fp8 and args.workload == "moe30b":
        # the bs=1 8K workload with the expert weights stored as E4M3 codes
        # and float32 row scales (the rest bf16)
        legs += [("fp8_experts", "moe30b_fp8")] + ([] if args.no_bs8 else [("fp8_experts_bs8", "moe30b_bs8_fp8")])
    if legs:
        for key, name in legs:
            wl8 = W.WORKLOADS[name]
            log(f"workload {wl8.name}: building inputs")
            n8 = max(8, args.steps // 2)
            eng8 = DecodeEngine(wl8, steps=args.warmup + n8 + 1, verbose=args.verbose)
            w8, k8, p8, r8 = time_steps(eng8, args.warmup, n8)
            m8 = step_metrics(wl8.model, wl8.batch, w8, k8, p8, r8, n8)
            m8["steps"] = n8
            m8["distinct_experts_per_layer"] = wl8.model.top_k if r8 is None else round(float(np.mean(
                [len(np.unique(r8[i].reshape(wl8.model.n_layers, -1)[l])) for i in range(n8)
                 for l in range(wl8.model.n_layers)])), 2)
            m8["config"] = {"workload": wl8.name, "batch": wl8.batch, "router_zipf": wl8.model.router_zipf,
                            "contexts": [W.context_length(wl8, b) for b in range(wl8.batch)]}
            if wl8.model.expert_fp8:
                m8["config"]["experts"] = "e4m3 codes + f32 row scales"
            out[key] = m8
            log(f"{key}: {m8['value']:.1f} tok/s, {m8['ms_per_step']:.3f} ms/step, "
                f"{m8['roofline']['frac']:.1%} of HBM SoL, {m8['distinct_experts_per_layer']} experts/layer")
            torch.cuda.synchronize()
            eng8.close()
            del eng8
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        try:
            out["cpu_baseline"] = cpu_baseline(wl)
        except Exception as e:  # the GPU figure stands on its own
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
