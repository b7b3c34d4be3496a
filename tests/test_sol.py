"""Speed-of-light accounting, pinned to the pages' own arithmetic.

The persistent decode megakernel pages (page 1, "Why decode leaves the GPU
idle"; page 3, "Where the bandwidth actually goes") put the bs=1 bound of the
30B / 3.3B-active model at about 470 tok/s: 6.6 GB of active bf16 weights plus
about 0.5 GB of KV at 8K context, over 3.35 TB/s.  292 tok/s is 62% of it and
185 tok/s is 39%.
"""
import math
import os

from persistent_moe_amd import sol
from persistent_moe_amd import workloads as W


def test_pages_speed_of_light_arithmetic():
    tok_s = sol.sol_tok_s(6.6e9 + 0.5e9, 1, bw=3.35e12)
    assert 465 < tok_s < 475
    assert abs(1e3 / tok_s - 2.1) < 0.05            # ~2.1 ms per step
    assert round(292 / 470, 2) == 0.62 and round(185 / 470, 2) == 0.39


def test_active_and_total_parameters_of_the_30b_model():
    cfg = W.MOE_30B
    active_bytes = sol.weight_bytes(cfg, 1, [cfg.top_k] * cfg.n_layers)
    active = active_bytes / 2
    assert abs(active / 3.3e9 - 1) < 0.02          # "3.3B active"
    total = sol.weight_bytes(cfg, 1, [cfg.n_experts] * cfg.n_layers) / 2 + cfg.vocab * cfg.d_model
    assert abs(total / 30.96e9 - 1) < 0.005        # ~30B total with an untied LM head


def test_step_bytes_of_the_bs1_8k_workload():
    cfg = W.MOE_30B
    nbytes = sol.step_bytes(cfg, [8192], [8] * 48)
    kv = 48 * 8193 * 2 * 4 * 128 * 2
    assert nbytes - sol.weight_bytes(cfg, 1, [8] * 48) == kv
    assert abs(nbytes / 7.33e9 - 1) < 0.01
    assert abs(sol.sol_tok_s(nbytes, 1) - 1092) < 10


def test_sliding_window_limits_kv():
    cfg = W.MOE_30B_SWA
    assert sol.visible_keys(cfg, 0, 262144) == 4096
    assert sol.visible_keys(cfg, 3, 262144) == 262145
    kv = sol.kv_bytes(cfg, [262144])
    assert kv == (12 * 262145 + 36 * 4096) * 2048


def test_fp8_expert_bytes_are_codes_plus_row_scales():
    """FP8 experts: one byte per weight and a float32 scale per output row
    (2I gate/up rows and d down rows per expert); the rest stays bf16."""
    from dataclasses import replace
    bf = W.MOE_30B
    f8 = replace(bf, expert_fp8=True)
    d, I, k = bf.d_model, bf.expert_inter, bf.top_k
    per_expert_bf16 = 3 * I * d * 2
    per_expert_fp8 = 3 * I * d + (2 * I + d) * 4
    diff = sol.layer_weight_bytes(bf, k) - sol.layer_weight_bytes(f8, k)
    assert diff == k * (per_expert_bf16 - per_expert_fp8)
    # 5.51 GB per bs=1 8K step with FP8 experts
    assert abs(sol.step_bytes(f8, [8192], [8] * 48) / 5.51e9 - 1) < 0.01


def test_bench_reports_traffic_only_for_the_sources_it_was_taken_with(tmp_path, monkeypatch):
    """The committed HBM-traffic summary carries the sha256 prefix of the
    kernel sources; with any source changed, bench.py reports no traffic."""
    import shutil
    import bench
    root = tmp_path / "repo"
    for f in bench.KERNEL_SOURCES + ["profiles/mk_persistent_moe30b_bs1_ctx8k_traffic.txt"]:
        (root / f).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), root / f)
    monkeypatch.setattr(bench, "ROOT", str(root))
    v = bench.measured_traffic("moe30b-bs1-ctx8k")
    assert v is not None and 7.3e9 < v < 7.5e9
    assert bench.measured_traffic("moe30b-bs8-ragged") is None
    with open(root / bench.KERNEL_SOURCES[1], "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("moe30b-bs1-ctx8k") is None
