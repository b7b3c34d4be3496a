"""Seeded random configurations, batch shapes and schedule options through
the host planner and the workspace sizing (no GPU): every call returns MK_OK
or a negative MK_E_* code and the process survives.  The calls run in a
child process, so that a crash shows as a failed test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r'''
import ctypes, random, sys
sys.path.insert(0, sys.argv[1])
from persistent_moe_amd import mk
from persistent_moe_amd import workloads as W
L = mk.load()
rng = random.Random(int(sys.argv[2]))
ints = [-2**31, -1, 0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 31, 32, 64, 100, 128, 129, 255, 256, 768, 1000, 1024,
        2047, 2048, 2049, 4096, 8192, 65536, 1 << 20, 2**31 - 1]
floats = [0.0, -1.0, 1e-6, 1e6, float("nan")]
seen = {}
for i in range(int(sys.argv[3])):
    p = float(sys.argv[4])
    base = mk.make_config(rng.choice([W.MOE_30B, W.TINY_MOE, W.DENSE_1B, W.MOE_30B_SWA, W.MOE_30B_FP8]),
                          rng.randint(1, 8))
    c = mk.mk_config()
    for name, _ in mk.mk_config._fields_:
        v = getattr(base, name)
        if rng.random() < p:
            v = rng.choice(floats) if name in ("rope_theta", "rms_eps") else rng.choice(ints)
        setattr(c, name, v)
    B = rng.choice([-1, 0, 1, 2, 8, 9])
    mb = rng.choice([-1, 0, 1, 5, 529, 1 << 20])
    o = mk.make_opts(rng.choice(list(mk.ORDER)), rng.choice(list(mk.LAUNCH)),
                     attn_split=rng.choice([-16, 0, 16, 64, 100, 384, 960, 5000]),
                     n_workgroups=rng.choice([-1, 0, 1, 7, 256, 257, 4096]), flags=rng.randint(0, 255),
                     moe_ug_pairs=rng.choice([-1, 0, 1, 24, 512, 513]),
                     moe_dn_rows=rng.choice([-1, 0, 1, 64, 2048, 5000]))
    nw = rng.choice([-3, 0, 1, 4, 7, 64, 256, 1024])
    nt, nc = ctypes.c_int32(), ctypes.c_int32()
    rc = L.mk_plan_schedule(ctypes.byref(c), B, mb, ctypes.byref(o), nw, None, 0, ctypes.byref(nt), ctypes.byref(nc))
    assert rc == 0 or -7 <= rc < 0, rc
    if rc == 0:
        assert nt.value > 0 and nc.value > 0
    L.mk_workspace_size(ctypes.byref(c), mb)
    seen[rc] = seen.get(rc, 0) + 1
print("codes", sorted(seen.items()))
'''


def _run(seed, n, p):
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, str(seed), str(n), str(p)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    return r.stdout


def test_planner_survives_random_configurations():
    out = _run(11, 3000, 0.25)
    assert "codes" in out


def test_planner_survives_mostly_valid_configurations():
    out = _run(12, 3000, 0.04)
    assert "(0," in out   # some of them plan
