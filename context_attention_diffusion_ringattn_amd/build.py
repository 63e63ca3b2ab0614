"""Build the HIP library ``libringattn.so`` in-tree for gfx950.

Usage: ``python -m context_attention_diffusion_ringattn_amd.build``.  Every
call compiles from source (hipcc cross-compiles; no GPU is needed).
``--sanitize`` builds a host-only AddressSanitizer + UndefinedBehaviorSanitizer
copy under ``_build/sanitize``; ``--sanitize-test`` also runs the CPU tests
against it.  ``--cycles`` builds a measurement copy under ``_build/cycles``
whose 8-wave kernel logs, per workgroup, the engine cycles and reference
ticks of its sweep (read by ``probes/sweep_cycles.py``).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libringattn.so")

SOURCES = ["api.cpp", "attn_pp.hip", "attn_w3.hip", "merge.hip", "noalloc.hip"]

# Packed fp32 VALU forms are disabled on purpose: the kernels are written with
# plain fp32 arithmetic and must not be lowered to v_pk_{add,mul,fma}_f32.
COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-fno-honor-nans",  # scores are finite or -inf, never NaN: lets fmaxf skip NaN canonicalisation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libringattn.so")


def _compile(hipcc: str, src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


PROBE_DIR = os.path.join(PKG_DIR, "probes")
PROBE_BIN = os.path.join(BUILD_DIR, "probes")
PROBES = ["issue_probe.hip", "lds_probe.hip"]


def _compile_probe(hipcc: str, src: str, verbose: bool) -> str:
    """A hardware probe (a stand-alone program, not part of the library)."""
    exe = os.path.join(PROBE_BIN, os.path.splitext(src)[0])
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(PROBE_DIR, src), "-o", exe]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling probe {src} failed:\n{res.stdout}{res.stderr}")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libringattn.so`` next to this file; also
    build the hardware probes under ``_build/probes``."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(PROBE_BIN, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBES)) as ex:
        probes = [ex.submit(_compile_probe, hipcc, p, verbose) for p in PROBES]
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose), SOURCES))
        for p in probes:
            p.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libringattn.so failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


CYCLES_DIR = os.path.join(BUILD_DIR, "cycles")
CYCLES_LIB = os.path.join(CYCLES_DIR, "libringattn.so")


def build_cycles(verbose: bool = False) -> str:
    """The library with the 8-wave kernel's sweep cycle log compiled in
    (RINGATTN_CYCLE_COUNTERS); the same kernels otherwise."""
    hipcc = _hipcc()
    os.makedirs(CYCLES_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(CYCLES_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON_FLAGS, "-DRINGATTN_CYCLE_COUNTERS", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compiling {src} (cycle counters) failed:\n{res.stdout}{res.stderr}")
        objs.append(obj)
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", CYCLES_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the cycle-counter library failed:\n{res.stdout}{res.stderr}")
    return CYCLES_LIB


SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libringattn.so")


def _clang() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ of the ROCm toolchain not found")


def build_sanitized(verbose: bool = False) -> str:
    """Build of every source whose host code (validation, chunk partition,
    layouts, launch planning, launch set-up) carries AddressSanitizer and
    UndefinedBehaviorSanitizer; the gfx950 code is compiled as usual and is
    not instrumented (the CPU tests never launch it).  The CPU tests run
    against it with ``RINGATTN_LIB`` pointing at it (``--sanitize-test``)."""
    hipcc = _hipcc()
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-Wall",
             "-fno-honor-nans", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", INCLUDE, "-I", CSRC]
    objs = []
    for src in SOURCES:
        obj = os.path.join(SANITIZE_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized compile of {src} failed:\n{res.stdout}{res.stderr}")
        objs.append(obj)
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", *objs, "-o", SANITIZE_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the sanitized library failed:\n{res.stdout}{res.stderr}")
    return SANITIZE_LIB


def sanitize_test() -> int:
    """Build the sanitized library and run the CPU test suite against it (the
    sanitizer runtime preloaded into the Python process; leak checking off,
    since the interpreter itself is not instrumented).  Returns pytest's exit
    status."""
    lib = build_sanitized()
    rt = subprocess.run([_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ)
    env["RINGATTN_LIB"] = lib
    env["LD_PRELOAD"] = (rt + " " + env["LD_PRELOAD"]).strip() if env.get("LD_PRELOAD") else rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    print("sanitized CPU tests:", " ".join(cmd), flush=True)
    rc = subprocess.run(cmd, env=env, cwd=ROOT).returncode
    if rc != 0:
        return rc
    # The instrumentation is live: an offsets buffer one entry short must be
    # reported as a heap-buffer-overflow by the sanitizer.
    probe = ("import ctypes, numpy as np; L = ctypes.CDLL(%r); a = np.zeros(8, dtype=np.int64); "
             "L.ringattn_chunk_offsets(ctypes.c_int64(4611), 8, 1, a.ctypes.data_as(ctypes.c_void_p))" % lib)
    res = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True)
    if res.returncode == 0 or "heap-buffer-overflow" not in res.stderr:
        print("the sanitizer did not report the planted overflow", file=sys.stderr)
        return 1
    print("sanitizer check: the planted heap-buffer-overflow was reported", flush=True)
    return 0


if __name__ == "__main__":
    if "--sanitize-test" in sys.argv:
        sys.exit(sanitize_test())
    if "--cycles" in sys.argv:
        print(build_cycles(verbose="-v" in sys.argv))
        sys.exit(0)
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
        sys.exit(0)
    path = build(verbose="-v" in sys.argv)
    print(path)
