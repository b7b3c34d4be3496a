"""Build the native parts in-tree: libmk.so (HIP, gfx950) and libpmgen.so (C).

``python -m persistent_moe_amd.build`` or ``build()``.  Always recompiles.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "lib")
GEN = os.path.join(PKG, "gen")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 arithmetic stays off (the compiler would otherwise form
    # v_pk_* fp32 ops from scalar float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_mk(verbose: bool = False) -> str:
    os.makedirs(LIB, exist_ok=True)
    out = os.path.join(LIB, "libmk.so")
    tmp = out + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + [os.path.join(CSRC, "mk_kernel.hip"), os.path.join(CSRC, "mk_host.cpp"),
                                 "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


def build_gen() -> str:
    out = os.path.join(GEN, "libpmgen.so")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           os.path.join(GEN, "pmgen.c"), "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_mk_host_sanitized(out: str) -> str:
    """libmk.so with AddressSanitizer and UndefinedBehaviorSanitizer on the
    host code only (the device code is built as usual), for checking the
    schedule builder, the simulator and the argument validation on the CPU.
    Load it with ``mk.load(out)`` in a process started with the clang ASan
    runtime preloaded (``LD_PRELOAD=.../libclang_rt.asan-x86_64.so``,
    ``ASAN_OPTIONS=detect_leaks=0``)."""
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
    cmd = ([HIPCC] + HIP_FLAGS + ["-Xarch_host", "-g"] + san +
           [os.path.join(CSRC, "mk_kernel.hip"), os.path.join(CSRC, "mk_host.cpp"), "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building the sanitized libmk.so")
    return out


def build(verbose: bool = False) -> None:
    build_gen()
    build_mk(verbose)


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        out = sys.argv[sys.argv.index("--host-sanitizers") + 1]
        print("built", build_mk_host_sanitized(out))
    else:
        build(verbose="-v" in sys.argv)
        print("built", os.path.join(LIB, "libmk.so"))
