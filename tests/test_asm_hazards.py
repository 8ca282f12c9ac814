"""The exact-path kernel's compiled gfx950 assembly has no unguarded hazard
around its inline-asm matrix products (see tests/asm_hazards.py).  Compiles
the kernel's source to device assembly on the host (hipcc cross-compiles; no
GPU needed) with the library's own flags."""

import os
import shutil
import subprocess

import pytest

from tests.asm_hazards import scan_function, split_kernels

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_context_block_amd", "csrc")


def _device_asm(tmp_path, source):
    from sparse_attention_context_block_amd import build

    hipcc = build.HIPCC
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "kernel.s"
    cmd = [hipcc, *build.FLAGS, *build.EXTRA.get(os.path.basename(source), []),
           "--cuda-device-only", "-S", source, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def test_scan_flags_planted_hazards():
    # a copy of a result one instruction after its product, and a VALU write of
    # an operand just before an inline-asm product, are both reported; the
    # same code with enough wait states is clean
    bad = "\n".join([
        ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]", ";;#ASMEND",
        "v_accvgpr_mov_b32 a20, a15",
        "v_mov_b32_e32 v5, 0",
        ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]", ";;#ASMEND",
        "s_endpgm"])
    found = scan_function(bad)
    assert any("touches" in m for _, m in found)
    assert any("written by the VALU" in m for _, m in found)
    good = "\n".join([
        ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]", ";;#ASMEND",
        "s_nop 7", "s_nop 7",
        "v_accvgpr_mov_b32 a20, a15",
        "v_mov_b32_e32 v5, 0",
        "s_nop 2",
        ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]", ";;#ASMEND",
        "s_endpgm"])
    assert scan_function(good) == []


def test_scan_follows_branches():
    text = "\n".join([
        ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        ";;#ASMEND", "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", ".LBB0_2:",
        "v_add_f32_e32 v30, v3, v4", "s_endpgm"])
    assert len(scan_function(text)) == 1


def test_exact_path_kernel_assembly_is_hazard_free(tmp_path):
    asm = _device_asm(tmp_path, os.path.join(CSRC, "isa_attn_w64.hip"))
    kernels = split_kernels(asm, r"_ZN3isa\w*attn_fwd_w64_kernel\w*")
    assert len(kernels) == 8  # b = 64 / 128, whole / partial tiles, first / fix-up launch
    for name, body in kernels.items():
        found = scan_function(body)
        assert not found, f"{name}: " + "; ".join(f"line {ln}: {m}" for ln, m in found[:5])
