"""Build ``libmuon_adamw.so`` (gfx950) from the HIP sources in ``csrc/``.

Usage: ``python -m adamw_optimizer_step_amd.build`` (or ``build()``). Objects
are compiled in parallel into ``_build/`` next to this file, then linked into
``libmuon_adamw.so`` in the package directory. Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmuon_adamw.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("MA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # elementwise stages are a bit-exact contract: one rounding per operation
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 arithmetic stays off (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# roctx, for the library's host-side ranges (rocprofv3 --marker-trace)
LINK = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]


# Per-kernel register budgets, checked on every build from the compiler's
# resource-usage remarks. The persistent GEMM runs two waves per SIMD; the
# AdamW update may run beside it on another stream, and one of its waves must
# fit in what the two leave of a SIMD's 512 VGPRs per lane (allocated in
# granules of 8), or a GEMM block cannot start on a CU where an AdamW wave is
# resident and waits for it to end. No kernel may use scratch memory.
VGPR_FILE, VGPR_GRANULE = 512, 8
GEMM_KERNEL, GEMM_WAVES_PER_SIMD = "ns_gemm_dma", 2
BESIDE_KERNEL = "k_adamw_lean"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]):\s+(\S+)")


def _alloc(n: int) -> int:
    return -(-max(n, 1) // VGPR_GRANULE) * VGPR_GRANULE


def parse_resources(text: str) -> dict:
    """{kernel: {"vgprs", "agprs", "scratch", "lds"}} from the text of
    ``-Rpass-analysis=kernel-resource-usage`` remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch", "LDS Size [bytes/block]": "lds"}
    for m in _REMARK.finditer(text):
        if m.group(1) == "Function Name":
            cur = out.setdefault(m.group(2), {})
        elif cur is not None:
            cur[keys[m.group(1)]] = int(m.group(2))
    return out


def check_resources(res: dict) -> list:
    """The budget violations in ``res`` (see parse_resources), as messages."""
    bad = [f"{k}: {v['scratch']} bytes of scratch per lane" for k, v in res.items() if v.get("scratch", 0)]
    beside = [v["vgprs"] + v.get("agprs", 0) for k, v in res.items() if BESIDE_KERNEL in k]
    if beside:
        room = VGPR_FILE - _alloc(max(beside))
        for k, v in res.items():
            if GEMM_KERNEL in k and GEMM_WAVES_PER_SIMD * _alloc(v["vgprs"] + v.get("agprs", 0)) > room:
                bad.append(f"{k}: {v['vgprs'] + v.get('agprs', 0)} VGPRs; {GEMM_WAVES_PER_SIMD} waves leave no room "
                           f"for a wave of {BESIDE_KERNEL} ({max(beside)})")
    return bad


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = (r.stderr or "").splitlines()
    res = parse_resources("\n".join(lines))
    # the remarks, each with its source excerpt, are not echoed
    err, skip = [], 0
    for l in lines:
        if "kernel-resource-usage" in l:
            skip = 2 if "Function Name" in l else 0
            continue
        if skip:
            skip -= 1
            continue
        if noise not in l:
            err.append(l)
    err = "\n".join(err)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj, res


# Host-side sanitizers for the planner and argument validation (api.hip, the
# host code of the C ABI): each flag applies to the host compilation only, so
# the device code is the same as in the product library. The result is a
# separate library for CPU-only tests, loaded with the ASan runtime preloaded.
HOST_SANITIZE = ["-Xarch_host -fsanitize=address", "-Xarch_host -fsanitize=undefined",
                 "-Xarch_host -fno-sanitize-recover=undefined", "-Xarch_host -fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "host_sanitized", "libmuon_adamw_hostsan.so")


def build_host_sanitized(verbose: bool = True) -> str:
    """``libmuon_adamw_hostsan.so``: the library with api.hip's host code built
    under AddressSanitizer and UndefinedBehaviorSanitizer (for CPU tests of the
    ABI; run it with the ASan runtime preloaded, see ``asan_runtime``)."""
    out = os.path.dirname(SAN_LIB)
    os.makedirs(out, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    for src in sources:
        if os.path.basename(src) == "api.hip":
            obj = os.path.join(out, "api.hip.o")
            flags = FLAGS + [f for pair in HOST_SANITIZE for f in pair.split()]
            r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            objs.append(obj)
        else:
            # the other sources' objects of the product build, when current
            obj = os.path.join(BUILD, os.path.basename(src) + ".o")
            fresh = os.path.exists(obj) and os.path.getmtime(obj) >= max(
                os.path.getmtime(f) for f in glob.glob(os.path.join(CSRC, "*")))
            objs.append(obj if fresh else _compile(src)[0])
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK, "-o", SAN_LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to LD_PRELOAD)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(_compile, sources))
    objs = [o for o, _ in done]
    res = {k: v for _, r in done for k, v in r.items()}
    with open(os.path.join(BUILD, "resources.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    bad = check_resources(res)
    if bad:
        raise RuntimeError("kernel resource budget exceeded:\n  " + "\n  ".join(bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({os.path.getsize(LIB)} bytes) from {len(sources)} sources")
    return LIB


if __name__ == "__main__":
    build_host_sanitized() if "--host-sanitized" in sys.argv else build()
