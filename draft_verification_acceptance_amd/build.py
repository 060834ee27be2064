"""Build libspecverify.so (HIP, gfx950) in-tree: python -m draft_verification_acceptance_amd.build"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["sv_api.hip", "sv_stats.hip", "sv_draw.hip", "sv_commit.hip", "sv_plan.hip", "sv_tree.hip", "sv_match.hip", "sv_probe.hip"]

# Packed fp32 VALU ops are kept out of the generated code (-packed-fp32-ops).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


# Per-file additions. sv_draw.hip: no atomic optimizer. It turns a one-lane atomic into a wave-wide one whose
# result is read into a scalar at once, which makes the wave wait for every load it has in flight; the draw
# claims its next batch of segments that way behind a trip's loads and uses the answer only at the batch's end.
FILE_FLAGS = {"sv_draw.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libspecverify)")


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (the device code is built as usual): for
# running the CPU tests of the host code (argument checks, workspace layout, the planner's host budget) under
# the sanitizers. Load it with the clang ASan runtime preloaded, see sanitize_env().
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g", "-shared-libasan"]
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libspecverify_san.so")


def sanitize_env() -> dict:
    """Environment for a process that loads SAN_LIB: the ASan runtime preloaded, leak checks off (the HIP
    runtime keeps allocations until exit), the binding pointed at the sanitized library."""
    cc = hipcc()
    rt = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True).stdout
    rt = rt.strip()
    if not os.path.exists(rt):
        llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(cc))), "lib", "llvm")
        import glob
        cands = glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
        rt = cands[0] if cands else rt
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SPECVERIFY_LIBRARY=SAN_LIB)
    return env


def build(verbose: bool = False, extra_flags: list[str] | None = None, sanitize: bool = False) -> str:
    build_dir = SAN_BUILD if sanitize else BUILD
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    flags = HIP_FLAGS + list(extra_flags or []) + (SAN_FLAGS if sanitize else [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *flags, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        cmd[3:3] = ["-fsanitize=address,undefined", "-shared-libasan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        # python -m draft_verification_acceptance_amd.build --sanitize [pytest args...]: build SAN_LIB, then run
        # the given CPU tests against it under ASan + UBSan
        print(build(verbose="-v" in sys.argv, sanitize=True))
        args = [a for a in sys.argv[1:] if a not in ("--sanitize", "-v")]
        if args:
            r = subprocess.run([sys.executable, "-m", "pytest", *args], env=sanitize_env(), cwd=ROOT)
            sys.exit(r.returncode)
    else:
        print(build(verbose="-v" in sys.argv))
