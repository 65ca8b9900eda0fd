"""Structural checks of the gfx950 code of the GEMM kernels (CPU only: hipcc
cross-compiles the device code to assembly; no GPU involved).

* Every direct global -> LDS copy (global_load_lds_dword[x4]) must take its
  64-bit base from SGPRs: the copies are issued from inline assembly with a
  wave-uniform base so that advancing a K step costs scalar adds only; a
  per-lane (VGPR) base would mean the compiler materialised the address in
  vector registers.
* No GEMM kernel spills to scratch or spills VGPRs (at most a few SGPRs go
  to VGPR lanes), and the LDS-tiled and streaming kernels fit two waves per
  SIMD (at most 256 registers per lane).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_expert_layer_gate_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")


def _asm(name, tmp_path):
    out = tmp_path / (name + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", os.path.join(CSRC, name), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm):
    """(name, metadata dict) for every kernel in the AMDGPU metadata block."""
    res = []
    for blk in re.findall(r"- \.agpr_count:.*?\.wavefront_size:\s+\d+", asm, re.S):
        md = dict(re.findall(r"\.(\w+):\s+([^\n]+)", blk))
        res.append((md.get("name", "?"), md))
    return res


@pytest.mark.parametrize("name", ["gemm_bf16_tiled.hip", "gemm_mx_tiled.hip"])
def test_lds_dma_copies_take_scalar_bases(name, tmp_path):
    asm = _asm(name, tmp_path)
    copies = re.findall(r"global_load_lds_dword(?:x4)?\s+([^\n]+)", asm)
    assert copies, "no direct global->LDS copies found"
    bad = [c for c in copies if re.match(r"v\d+,\s*v\[", c)]
    assert not bad, f"{len(bad)} of {len(copies)} copies take a VGPR base: {bad[:3]}"


@pytest.mark.parametrize("name", ["gemm_bf16_tiled.hip", "gemm_mx_tiled.hip",
                                  "gemm_bf16_stream.hip"])
def test_gemm_kernels_no_spill_two_waves(name, tmp_path):
    ks = _kernels(_asm(name, tmp_path))
    assert ks
    for kname, md in ks:
        assert int(md["vgpr_spill_count"]) == 0, kname
        # SGPRs spilled into VGPR lanes (v_writelane / v_readlane) cost no
        # memory traffic; a handful is tolerated, scratch never
        assert int(md["sgpr_spill_count"]) <= 4, kname
        assert int(md["private_segment_fixed_size"]) == 0, kname
        total = int(md["vgpr_count"])
        assert total <= 256, f"{kname}: {total} registers per lane"
