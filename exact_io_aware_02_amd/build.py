"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python exact_io_aware_02_amd/build.py [--verbose] [--resource-usage] [--host-sanitizers]

(run as a script: importing the package would load the library first)

Every source is compiled on each call (hipcc cross-compiles without a GPU).
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_bf16_asm.hip", "fa_fwd_f32.hip", "fa_decode.hip",
           "fa_bwd_bf16.hip", "fa_probe.hip"]
# generated before compiling: the assembly of the 64-rows-per-wavefront
# forward's tile loop (fa_fwd_bf16_asm.hip includes it)
GENERATED = os.path.join(CSRC, "fa_fwd_asm_d128.inc")
# NaN inputs are outside the contract of the bf16 kernels; without NaN
# semantics fmaxf needs no canonicalisation and fuses into v_max3_f32.
# Infinities stay honoured (masked scores are -inf).
PER_SOURCE_FLAGS = {
    "fa_fwd_bf16.hip": ["-fno-honor-nans"],
    "fa_fwd_bf16_asm.hip": ["-fno-honor-nans"],
    "fa_decode.hip": ["-fno-honor-nans"],
    "fa_bwd_bf16.hip": ["-fno-honor-nans"],
}

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32
# (the host pass prints a harmless "not a recognized feature" warning).
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        ln for ln in p.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln
    )
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, resource_usage=False):
    """Compile every source and link libfa.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    _run([sys.executable, os.path.join(PKG, "gen_fwd_asm.py"), GENERATED], verbose)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, *PER_SOURCE_FLAGS.get(src, []), *extra, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose or resource_usage), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    _check_undefined(tmp)
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(OBJDIR, "host_sanitizers")
SAN_LIB = os.path.join(SAN_DIR, "libfa_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only (the
# device code of the same file is compiled as usual)
SAN_FLAGS = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def build_host_sanitized(verbose=False):
    """libfa_san.so: the host dispatch (fa_api.hip: argument checks, overlap
    tests, planners, the workspace and scratch maps) compiled with ASan and
    UBSan, linked with the objects of the ordinary build (built first if
    missing).  Load it with the ASan runtime preloaded (asan_runtime())."""
    hipcc = _hipcc()
    objs = [os.path.join(OBJDIR, src.replace(".hip", ".o")) for src in SOURCES if src != "fa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    os.makedirs(SAN_DIR, exist_ok=True)
    api = os.path.join(SAN_DIR, "fa_api.o")
    _run([hipcc, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "fa_api.hip"), "-o", api], verbose)
    tmp = SAN_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", api, *objs, "-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def asan_runtime():
    """Path of the compiler's shared ASan runtime (to preload into Python)."""
    p = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def _check_undefined(path):
    """Fail if the host pass dropped a kernel launch stub (the library would
    then not load)."""
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm is None:
        return
    out = subprocess.run([nm, "-D", "--undefined-only", path], stdout=subprocess.PIPE, text=True).stdout
    missing = [ln.split()[-1] for ln in out.splitlines() if "device_stub" in ln]
    if missing:
        raise RuntimeError("libfa.so references undefined kernel stubs: " + ", ".join(missing))


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true", help="print VGPR/LDS usage per kernel")
    ap.add_argument("--host-sanitizers", action="store_true",
                    help="also build libfa_san.so (host dispatch with ASan + UBSan)")
    a = ap.parse_args()
    print(build(verbose=a.verbose, resource_usage=a.resource_usage))
    if a.host_sanitizers:
        print(build_host_sanitized(verbose=a.verbose))
    sys.exit(0)
