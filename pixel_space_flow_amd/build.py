"""Build libpsf_gen.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python pixel_space_flow_amd/build.py        # or __graft_entry__.build()
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpsf_gen.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["gemm.hip", "attention.hip", "elementwise.hip", "moe.hip", "backward.hip", "skinny.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # keep the compiler from emitting packed fp32 VALU ops
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")


def _resources(remarks: str):
    """(kernel symbol, VGPRs, AGPRs, scratch bytes per lane) from the compiler's
    kernel-resource-usage remarks."""
    out, cur = [], None
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        key, _, val = body.partition(":")
        val = val.strip()
        if key == "Function Name":
            cur = [val, 0, 0, 0]
            out.append(cur)
        elif cur is not None and key == "VGPRs":
            cur[1] = int(val)
        elif cur is not None and key == "AGPRs":
            cur[2] = int(val)
        elif cur is not None and key.startswith("ScratchSize"):
            cur[3] = int(val)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    # per-kernel register and scratch use of this build (a spill shows as scratch > 0)
    with open(RESOURCES, "w") as f:
        for _, res in done:
            for name, v, a, sc in res:
                f.write(f"{name} vgprs={v} agprs={a} scratch={sc}\n")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


SAN_DIR = os.path.join(BUILD_DIR, "host_asan")
SAN_OUT = os.path.join(BUILD_DIR, "libpsf_gen_host_asan.so")
# the host pass instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; the device code
# is built as usual (no GPU sanitizer)
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Wno-unused-result"]


def _sources_stamp(flags) -> str:
    import hashlib
    h = hashlib.sha256(" ".join(flags).encode())
    for f in sorted(os.listdir(CSRC)):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    h.update(open(os.path.join(HERE, "..", "include", "psf_gen.h"), "rb").read())
    h.update(open(os.path.join(HERE, "..", "include", "psf_gen_ops.h"), "rb").read())
    return h.hexdigest()


def build_host_sanitized(verbose: bool = True) -> str:
    """The library with its host code (the C ABI, argument validation, workspace layout,
    launchers) built with AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests of
    the host-side checks; rebuilt only when a source changed.  Load it with clang's ASan runtime
    preloaded (libclang_rt.asan-x86_64.so)."""
    stamp = _sources_stamp(SAN_FLAGS)
    stamp_file = SAN_OUT + ".stamp"
    if os.path.exists(SAN_OUT) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return SAN_OUT
    os.makedirs(SAN_DIR, exist_ok=True)

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *SAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host) failed for {src}:\n{r.stderr}")
        return obj
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", *objs, "-o", SAN_OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized host) failed:\n{r.stderr}")
    with open(stamp_file, "w") as f:
        f.write(stamp)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "host-asan":
        build_host_sanitized()
    else:
        build()
    sys.exit(0)
