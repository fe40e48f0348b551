"""Builds librn_retention.so in-tree with hipcc for gfx950.

    python linear_recurrent_sequence_rn_amd/build.py

(Run as a script: importing the package loads the library, which may not exist yet.)

Every HIP source under csrc/ is compiled to an object under _build/ and linked into
linear_recurrent_sequence_rn_amd/librn_retention.so. Always recompiles.

build(sanitize=True, lib=path) makes a copy whose host code is built with
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged), for running
the host-side tests under the sanitizers; the process that loads it must preload the
ASan runtime (sanitizer_runtime() names it).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "librn_retention.so"
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # packed fp32 instructions stay off in every HIP object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs: the kernels scale, convert and store most of them
    # with VALU instructions, which would otherwise copy them out of AGPRs first
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + [
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g"]


def _compile(src: Path, build_dir: Path = BUILD, extra=()) -> Path:
    obj = build_dir / (src.stem + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-x", "hip", "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stderr}")
    return obj


def sanitizer_runtime() -> str:
    """Path of the ASan runtime of the compiler that builds the sanitized library."""
    clang = Path(HIPCC).resolve().parent.parent / "llvm" / "bin" / "clang"
    if not clang.exists():
        clang = Path("/opt/rocm/llvm/bin/clang")
    r = subprocess.run([str(clang), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False, lib: Path = LIB) -> Path:
    build_dir = BUILD / "sanitize" if sanitize else BUILD
    build_dir.mkdir(parents=True, exist_ok=True)
    srcs = sources()
    extra = SANITIZE if sanitize else ()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    lib = Path(lib)
    tmp = lib.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(
        ["-Xarch_host", "-shared-libsan"] if sanitize else []), "-o", str(tmp), *map(str, objs),
        "-lrocblas"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
