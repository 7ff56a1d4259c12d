"""Build libqurl_w8a8.so for gfx950 in-tree with hipcc.

Usage: python -m w8a8_gemm_rl_amd.build   (or __graft_entry__.build()).

Each HIP source is compiled to an object in ``_build/`` (in parallel), then the
objects are linked into ``w8a8_gemm_rl_amd/libqurl_w8a8.so``. The library is
rebuilt from scratch on every call. Flags: correctly rounded fp32 division and
IEEE denormals are hipcc's defaults and must stay so (the quantized codes
depend on them); packed-fp32 instruction selection is switched off.

The compiler's per-kernel resource report is read back, and the build fails
if any kernel keeps registers in scratch memory: every kernel here is sized
to fit its register budget, and a spill (for instance from a change that
keeps more values live across a GEMM's K loop) silently costs a large part
of its speed.
"""

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqurl_w8a8.so")
SOURCES = ["quant_kernels.hip", "producer_kernels.hip", "gemm_kernels.hip", "gemm_plan.hip",
           "acr_kernels.hip", "mx_kernels.hip", "probe_kernels.hip", "small_m_kernels.hip", "qr_api.hip",
           "qr_noalloc.hip"]
# Per-source flags: the fused producers fix the order of their fp32 roundings,
# so no multiply-add may be contracted there.
EXTRA = {"producer_kernels.hip": ["-ffp-contract=off"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _spills(report):
    """(kernel, scratch bytes per lane) for every kernel of a resource report
    that uses scratch; the report's other remarks are dropped."""
    bad, name = [], None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def _strip_remarks(out):
    keep, skip = [], False
    for line in out.splitlines():
        if "-Rpass-analysis=kernel-resource-usage" in line:
            skip = True  # the remark's source excerpt follows
            continue
        if skip and (line.startswith(" ") or not line.strip()):
            continue
        skip = False
        keep.append(line)
    return "\n".join(keep)


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        out = _run([HIPCC, *CFLAGS, *EXTRA.get(SOURCES[i], []), "-Rpass-analysis=kernel-resource-usage",
                    "-c", src, "-o", objs[i]])
        bad = _spills(out)
        if bad:
            raise RuntimeError(f"{SOURCES[i]}: kernels spill registers to scratch memory: "
                               + ", ".join(f"{n} ({b} bytes per lane)" for n, b in bad))
        return _strip_remarks(out)

    jobs = jobs or min(len(SOURCES), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the whole
# library (argument validation, planning, error reporting, the launchers'
# host code); device code is compiled as usual. For CPU tests only: it lives
# in _build/sanitize/, never next to the package, and needs the sanitizer
# runtime preloaded into the process that loads it.
SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libqurl_w8a8_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")


def sanitizer_runtime():
    """Path of clang's shared AddressSanitizer runtime (to preload)."""
    out = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("clang's shared AddressSanitizer runtime was not found")
    return out


def build_sanitized(jobs=None):
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = [os.path.join(SAN_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        return _run([HIPCC, *CFLAGS, *EXTRA.get(SOURCES[i], []), *SAN_HOST_FLAGS, "-c", src, "-o",
                     objs[i]])

    jobs = jobs or min(len(SOURCES), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(compile_one, range(len(SOURCES))))
    # the link is a host link of HIP objects (each embeds its device code)
    _run([CLANGXX, "-shared", "-fPIC", "-shared-libasan", "-fsanitize=address,undefined", *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", SAN_LIB])
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitize":
        print(build_sanitized())
    else:
        build(verbose=True)
    sys.exit(0)
