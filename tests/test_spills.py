"""Zero-spill audit of every kernel the library builds (CPU only: compile-time facts).

The register budget of each kernel is fixed by its tile and K slice, never by
K; the audit checks the compiler's resource report, the kernel descriptors and
the assembly of our own build for any scratch use, and a deliberately
spilling kernel shows that the audit can fail.
"""

import json
import os
import subprocess

import pytest

from tiled_shared_memory_amd import build as B


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(B.REPORT) or not os.path.exists(B.LIBRARY):
        B.build_library(verbose=False)
    return json.load(open(B.REPORT))


def test_every_kernel_is_spill_free(report):
    private = report["private_segment_fixed_size"]
    kernels = [k for k in report["kernels"] if k["name"] in private]
    assert kernels, "no kernels in the resource report"
    assert B.audit(kernels, private, []) == []
    for k in kernels:
        assert int(k["ScratchSize [bytes/lane]"]) == 0
        assert int(k["VGPRs Spill"]) == 0 and int(k["SGPRs Spill"]) == 0
        assert private[k["name"]] == 0


def test_lds_fits_the_cu(report):
    private = report["private_segment_fixed_size"]
    for k in report["kernels"]:
        if k["name"] in private:
            assert int(k["LDS Size [bytes/block]"]) <= 160 * 1024


def test_every_kernel_family_is_built(report):
    names = " ".join(k["name"] for k in report["kernels"])
    assert "gemm_masked_kernel" in names
    assert "gemm_tile_kernel" in names


SPILLER = r"""
#include <hip/hip_runtime.h>
// Deliberately needs far more registers than a lane has: a dynamically indexed
// private array forces scratch memory.
__global__ void spill_on_purpose(float *out, const int *idx) {
  float big[2048];
  for (int i = 0; i < 2048; ++i) big[i] = out[i * 64 + threadIdx.x];
  out[threadIdx.x] = big[idx[threadIdx.x] & 2047];
}
"""


def test_audit_flags_a_spilling_kernel(tmp_path):
    src = tmp_path / "spill.hip"
    src.write_text(SPILLER)
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-c", str(src), "-o", str(tmp_path / "s.o"),
                        "-Rpass-analysis=kernel-resource-usage", "-save-temps"], cwd=tmp_path, capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    kernels = B.parse_remarks(r.stderr + r.stdout)
    asm = open(tmp_path / f"spill-hip-amdgcn-amd-amdhsa-{B.ARCH}.s").read()
    private = B.parse_private_segments(asm)
    bad = B.audit([k for k in kernels if k["name"] in private], private, B.scratch_instructions(asm))
    assert bad, "the audit let a scratch-using kernel through"
    assert any("ScratchSize" in b or "private_segment" in b for b in bad)
