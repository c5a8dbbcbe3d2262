"""Compile the HIP sources under csrc/ into the in-tree shared library libfa.so (gfx950).

It also links libfa_serial.so, a debug build whose bf16 forward runs the serial
form of its loop (FA_SERIAL_PIPELINE: one tile at a time, one LDS slot, full
barriers) and must agree with libfa.so bit for bit; tests load it next to the
product library."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
LIB_SERIAL = os.path.join(PKG, "libfa_serial.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "scratch.hip", "calib.hip", "attn_f32.hip", "attn_bf16.hip", "quant_fp8.hip", "attn_fp8.hip", "merge.hip", "attn_bwd.hip"]
EXTRA = {}  # per-source extra flags

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, defines: tuple = ()) -> str:
    tag = "".join("_" + d.split("=")[0].lower() for d in defines)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *("-D" + d for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(lib: str, objs: list) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


SERIAL_SOURCE = "attn_bf16.hip"


def build(jobs: int = 6, verbose: bool = True) -> str:
    """Compile every source (always), link libfa.so and the debug libfa_serial.so;
    returns the product library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs_list = [(src, ()) for src in SOURCES] + [(SERIAL_SOURCE, ("FA_SERIAL_PIPELINE=1",))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs_list))
    prod = objs[: len(SOURCES)]
    _link(LIB, prod)
    serial = [objs[-1] if src == SERIAL_SOURCE else o for src, o in zip(SOURCES, prod)]
    _link(LIB_SERIAL, serial)
    if verbose:
        print(f"built {LIB} and {LIB_SERIAL}")
    return LIB


if __name__ == "__main__":
    build()
