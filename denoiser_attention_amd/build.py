"""Build libtt.so (and the roof probes, libtt_probes.so) in-tree with hipcc for gfx950.

    python -m denoiser_attention_amd.build        # or: python denoiser_attention_amd/build.py

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into denoiser_attention_amd/libtt.so with only
the tt_* C entry points exported.  Object files go to _build/ at the repo root.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtt.so")
PROBE_LIB = os.path.join(PKG, "libtt_probes.so")
# Per-kernel register, spill, scratch and LDS figures reported by the compiler
# for the last build (read by the CPU tests that guard against spills).
RESOURCES = os.path.join(BUILD, "kernel_resources.json")


def device_asm(src: str) -> str:
    """Path of the gfx950 assembly the last build wrote for a .hip source (read
    by the CPU tests that check hazards the compiler cannot see through inline
    asm)."""
    return os.path.join(BUILD, os.path.basename(src) + ".s")

SOURCES = ["tt_api.cpp", "attn_mfma.hip", "attn_shuffle.hip", "unmask.hip", "lmhead.hip"]
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # Keep hipcc from selecting packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
    # Per-kernel resource remarks (registers, spills, scratch, LDS, occupancy).
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark:\s+(Function Name|[A-Za-z][A-Za-z /\[\]]*?): (\S+) \[-Rpass-analysis")
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
           "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "waves_per_simd",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}


def parse_resources(text: str) -> dict:
    """Kernel name -> resource figures, from the compiler's resource remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            cur[_FIELDS[key]] = int(val) if val.isdigit() else val
    return out


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libtt")
    return exe


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    resources = parse_resources("\n".join(lines))
    if src.endswith(".hip"):
        # The device assembly of the same source, for the hazard checks.
        acmd = [hipcc(), *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o",
                device_asm(src)]
        a = subprocess.run(acmd, capture_output=True, text=True)
        if a.returncode != 0:
            raise RuntimeError(f"hipcc -S failed on {src}:\n{a.stdout}{a.stderr}")
    # Everything but the resource remarks (and the source excerpts under them).
    msg = "\n".join(l for l in lines if "kernel-resource-usage" not in l and not re.match(r"^\s+(\d+ \||\|)", l))
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj, resources


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


# A plain C99 client of the C ABI (include/tt.h + the HIP runtime, no Python),
# built next to its source and run by the tests.
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "tt_c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c", "tt_c_client")


def c_client_command(src: str, out: str) -> list:
    """gcc command that builds a C99 program against include/tt.h and libtt.so
    (found at run time next to the program's relative path to the package)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C ABI client")
    rel = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    return [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", INCLUDE, "-I", os.path.join(rocm, "include"), src, "-o", out,
            "-L", PKG, "-ltt", f"-Wl,-rpath,$ORIGIN/{rel}",
            "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]


def _build_c_client(verbose):
    if (shutil.which("gcc") or shutil.which("cc")) is None:
        print("build: no C compiler; the C ABI client is not built (its tests skip)", flush=True)
        return
    tmp = C_CLIENT + ".tmp"
    cmd = c_client_command(C_CLIENT_SRC, tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, C_CLIENT)


def build(verbose: bool = False) -> str:
    """Compile every source and link libtt.so and libtt_probes.so, then the C
    client of the ABI.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        done = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    objs = {s: o for s, (o, _) in done.items()}
    resources = {s: res for s, (_, res) in done.items()}
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    _build_c_client(verbose)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
