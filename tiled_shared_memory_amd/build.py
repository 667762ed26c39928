"""Build the gfx950 HIP library and audit every kernel for scratch use.

``build_library()`` compiles each ``csrc/*.hip`` with hipcc for gfx950 only,
links ``libtsm_gemm.so`` into this package directory, and records the compiler's
per-kernel resource usage.  The audit then requires, for every kernel:

  * ScratchSize 0 bytes/lane, VGPRs Spill 0, SGPRs Spill 0 (compiler remarks),
  * ``.private_segment_fixed_size: 0`` in the kernel descriptor metadata,
  * no ``scratch_`` instruction in the generated assembly.

This is the gfx950 form of the zero-spill rule: on "The PTSS Cliff" page
(section "The Cliff: 345 KB Spill, 256 KB Cap") a schedule whose spill exceeds
the per-thread scratch cap does not even build; here the register budget is
fixed by the tile and the loop slice, and any spill fails the build outright.
"""

from __future__ import annotations

import glob
import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libtsm_gemm.so")
REPORT = os.path.join(BUILD_DIR, "resource_usage.json")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

HIPFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # packed float32 VALU ops stay off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
    "-save-temps",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]

_REMARK = re.compile(r"remark: (?P<file>[^:]+):\d+:\d+:\s+(?P<key>[^:]+?):\s*(?P<val>.*?)\s*\[-Rpass-analysis")


def parse_remarks(text: str):
    """Per-kernel resource records from ``-Rpass-analysis=kernel-resource-usage`` output."""
    kernels = []
    cur = None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group("key").strip(), m.group("val").strip()
        if key == "Function Name":
            cur = {"name": val, "file": os.path.basename(m.group("file"))}
            kernels.append(cur)
        elif cur is not None:
            cur[key] = val
    return kernels


def parse_private_segments(asm_text: str):
    """``.private_segment_fixed_size`` of every kernel in an assembly file."""
    sizes = {}
    name = None
    for line in asm_text.splitlines():
        s = line.strip()
        if s.startswith(".name:"):
            name = s.split(":", 1)[1].strip()
        elif s.startswith(".private_segment_fixed_size:") and name is not None:
            sizes[name] = int(s.split(":", 1)[1])
    return sizes


def scratch_instructions(asm_text: str):
    return [ln.strip() for ln in asm_text.splitlines() if re.match(r"\s*scratch_\w+", ln)]


def audit(kernels, private_sizes=None, scratch_ops=None):
    """List of human-readable violations (empty = every kernel is spill free)."""
    bad = []
    for k in kernels:
        for key in ("ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill"):
            if key not in k:
                bad.append(f"{k['name']}: no '{key}' remark")
            elif int(k[key]) != 0:
                bad.append(f"{k['name']}: {key} = {k[key]}")
        if k.get("Dynamic Stack", "False") != "False":
            bad.append(f"{k['name']}: dynamic stack")
    for name, size in (private_sizes or {}).items():
        if size != 0:
            bad.append(f"{name}: .private_segment_fixed_size = {size}")
    for op in scratch_ops or []:
        bad.append(f"scratch instruction: {op}")
    return bad


def _compile(src: str, verbose: bool):
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD_DIR, base + ".o")
    cmd = [HIPCC, *HIPFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, cwd=BUILD_DIR, capture_output=True, text=True)
    log = r.stdout + r.stderr
    with open(os.path.join(BUILD_DIR, base + ".log"), "w") as fh:
        fh.write(" ".join(cmd) + "\n" + log)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{log[-4000:]}")
    if verbose:
        print(f"[build] compiled {base}.hip", flush=True)
    return obj, log, base


def build_library(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile and link the library; raise if any kernel uses scratch memory."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(sources), 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), sources))
    objs = [r[0] for r in results]
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, cwd=BUILD_DIR, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIBRARY)

    kernels, private, scratch = [], {}, []
    for _, log, base in results:
        kernels.extend(parse_remarks(log))
        for asm in glob.glob(os.path.join(BUILD_DIR, f"{base}-hip-amdgcn-amd-amdhsa-{ARCH}.s")):
            text = open(asm).read()
            private.update(parse_private_segments(text))
            scratch.extend(scratch_instructions(text))
    report = {"arch": ARCH, "kernels": kernels,
              "private_segment_fixed_size": private}
    with open(REPORT, "w") as fh:
        json.dump(report, fh, indent=1)
    bad = audit([k for k in kernels if _is_kernel(k, private)], private, scratch)
    if bad:
        raise RuntimeError("register budget violated (spills or scratch):\n  " + "\n  ".join(bad))
    if verbose:
        print(f"[build] {LIBRARY}: {len(private)} kernels, 0 spills, 0 scratch", flush=True)
    return LIBRARY


def _is_kernel(rec, private):
    # the remark covers device functions too; kernels are the ones with a descriptor
    return rec["name"] in private if private else True


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)
    if os.path.exists(LIBRARY):
        os.remove(LIBRARY)


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
