"""Build step: compile the HIP sources into the in-tree C-ABI library.

``python bwd_dyt_forward_amd/build.py`` (or ``build()``) runs hipcc for gfx950
and writes ``bwd_dyt_forward_amd/libdyt.so``. Cross-compiling needs no GPU.
"""
from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_NAME = "libdyt.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# Host logic and the kernel instances per x dtype and direction: separate
# translation units, compiled in parallel.
SOURCES = [os.path.join(CSRC, "dyt_api.hip")] + [
    os.path.join(CSRC, f"dyt_launch_{d}_{t}.hip") for d in ("fwd", "bwd") for t in ("f32", "bf16", "f16")]
DEPENDS = SOURCES + [os.path.join(CSRC, f) for f in (
    "dyt_kernels.hpp", "dyt_math.hpp", "dyt_launch.hpp", "dyt_launch_impl.hpp",
    "dyt_tune_table.inc")] + [os.path.join(INCLUDE, "dyt.h")]
# Reference streaming kernels for bench.py's measured ceilings (not part of
# the DyT ABI; nothing in the package loads them).
STREAM_REF_SOURCE = os.path.join(CSRC, "stream_ref.hip")
STREAM_REF_PATH = os.path.join(PKG_DIR, "libdyt_streamref.so")

ARCH = "gfx950"

# No fast-math and no denormal flushing: float32 subnormals must survive
# (x subnormal with alpha = inf gives +-gamma + beta, not NaN). Packed fp32
# VALU ops are disabled for the device pass.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# parallel compilations (at most 16: the share of a GPU machine's CPUs)
JOBS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


# The library embeds BUILD_ID_MARK followed by the 16 hex digits of
# source_hash() as it was at build time (and returns them from
# dyt_build_id()), so a library can be matched to the sources it came from.
BUILD_ID_MARK = b"DYT_BUILD_ID="


def source_hash(extra_flags=()) -> str:
    """Hash of every source the library is built from (kernels, launch and
    host code, the tile table, the header) with comments and blank space
    removed, and of the compiler flags (plus the extra flags of a variant
    build): two trees with the same hash build the same code."""
    h = hashlib.sha256()
    for p in DEPENDS:
        with open(p) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(os.path.basename(p).encode() + b"\0")
        h.update(" ".join(src.split()).encode() + b"\0")
    h.update(" ".join([*HIPCC_FLAGS, *extra_flags]).encode())
    return h.hexdigest()[:16]


def built_id(path: str = LIB_PATH) -> str | None:
    """The build id embedded in a built library (read from the file, without
    loading it), or None if the file or the id is missing."""
    try:
        with open(path, "rb") as f:
            data = f.read()
    except OSError:
        return None
    at = data.find(BUILD_ID_MARK)
    if at < 0:
        return None
    hexid = data[at + len(BUILD_ID_MARK): at + len(BUILD_ID_MARK) + 16]
    return hexid.decode("ascii", "replace")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DyT library needs ROCm's hipcc to build")


# Object files of cached builds (build(cache=True)), keyed by the content of
# the source, of every header and of the flags.
OBJ_CACHE = os.path.join(PKG_DIR, "_build")


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None, verbose: bool = False,
          with_stream_ref: bool = True, cache: bool = False) -> str:
    """Compile the library (and, by default, the reference streaming kernels
    next to the default library path); returns the library's path. Always
    recompiles every source, unless cache=True, which reuses the object of
    a translation unit whose source, headers and flags are unchanged. Only
    the host translation unit carries the build id."""
    extra = list(extra_flags or [])
    per_source = {SOURCES[0]: [f'-DDYT_BUILD_ID="{source_hash(extra)}"']}
    _compile(out, SOURCES, extra, verbose, per_source, OBJ_CACHE if cache else None)
    if with_stream_ref and out == LIB_PATH:
        _compile(STREAM_REF_PATH, [STREAM_REF_SOURCE], None, verbose)
    return out


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)


def _object_key(src: str, flags: list[str]) -> str:
    h = hashlib.sha256()
    for p in [src] + [d for d in DEPENDS if not d.endswith(".hip")]:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:20]


def _compile(out: str, sources: list[str], extra_flags: list[str] | None, verbose: bool,
             per_source: dict | None = None, cache_dir: str | None = None) -> None:
    """Each source to an object (in parallel), then one shared library."""
    flags = [*HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *(extra_flags or [])]
    per_source = per_source or {}
    with tempfile.TemporaryDirectory(prefix="dyt_build_") as tmpdir:
        jobs = []
        objs = []
        for src in sources:
            f = [*flags, *per_source.get(src, [])]
            name = os.path.basename(src)
            if cache_dir:
                os.makedirs(cache_dir, exist_ok=True)
                obj = os.path.join(cache_dir, f"{name}-{_object_key(src, f)}.o")
                if not os.path.exists(obj):
                    jobs.append((f, src, obj))
            else:
                obj = os.path.join(tmpdir, name + ".o")
                jobs.append((f, src, obj))
            objs.append(obj)

        def one(job):
            f, src, obj = job
            tmp_obj = obj + ".tmp" if cache_dir else obj
            _run([hipcc(), *f, "-c", "-o", tmp_obj, src], verbose)
            if cache_dir:
                os.replace(tmp_obj, obj)

        if jobs:
            with ThreadPoolExecutor(max_workers=min(JOBS, len(jobs))) as ex:
                list(ex.map(one, jobs))
        tmp = out + ".tmp"
        _run([hipcc(), *flags, "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, out)


def is_stale(path: str = LIB_PATH, extra_flags=()) -> bool:
    """True if the library is missing or was built from other sources or
    flags than the current ones (by content, not by file times)."""
    return built_id(path) != source_hash(extra_flags)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
