"""The generated gfx950 code of the GEMM kernels: no register spills in the K loops.

A spill in the K loop is a scratch access in the middle of the DMA pipeline:
its wait (vmcnt) also waits for every load in flight, and one such reload
has made a kernel 40% slower. Register allocation at 256 VGPRs + 256 AGPRs
is close to the edge, so a harmless-looking source change can cause one.
This test compiles the kernel source to gfx950 assembly (no GPU needed) and
checks every loop that holds one K step's MFMAs of the default bf16 engine.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_optimizer_step_muon_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _k_step_loops(asm: str, kernel_pattern: str, mfma_per_step: int, innermost: bool = False):
    """(kernel, loop length, MFMAs, scratch accesses) of the loops of the
    matching kernels that hold exactly one K step's MFMAs; with innermost, only
    those that hold no other loop's backward branch."""
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*:", l) and re.search(kernel_pattern, l)]
    out = []
    for st in starts:
        end = next(i for i in range(st, len(lines)) if "s_endpgm" in lines[i])
        body = lines[st:end]
        labels = {}
        for i, l in enumerate(body):
            m = re.match(r"^(\.LBB\d+_\d+):", l)
            if m:
                labels[m.group(1)] = i
        for i, l in enumerate(body):
            m = re.search(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", l)
            if not (m and m.group(1) in labels and labels[m.group(1)] < i):
                continue
            a = labels[m.group(1)]
            seg = body[a:i + 1]
            nm = sum(1 for x in seg if "v_mfma" in x)
            if nm != mfma_per_step:
                continue
            if innermost and any(re.search(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", x) and
                                 labels.get(re.search(r"(\.LBB\d+_\d+)\s*$", x.strip()).group(1), i + 1) < a + k
                                 for k, x in enumerate(seg[:-1])
                                 if re.search(r"s_(?:cbranch_\w+|branch)\s+\.LBB\d+_\d+\s*$", x.strip())):
                continue
            ns = sum(1 for x in seg if re.search(r"\bscratch_(load|store)", x))
            out.append((body[0].split(":")[0], i - a, nm, ns))
    return out


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "muon_kernels.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "muon_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_default_engine_k_loops_do_not_spill(kernel_asm):
    # Engine4<QK, 64, 2>: K step 64 = 4 sub-steps of 16 MFMAs.
    loops = _k_step_loops(kernel_asm, r"phase_kernel4INS_7Engine4ILb[01]ELi64ELi2EEE", 64)
    kernels = {k for k, _, _, _ in loops}
    assert len(kernels) == 6, ("expected the gram (with and without split-K pieces), square, update and "
                               f"last-update kernels (bf16 and fp32 W), found {kernels}")
    bad = [(k[-40:], n, s) for k, n, _, s in loops if s]
    assert not bad, f"K-step loops with scratch accesses (kernel, length, accesses): {bad}"


def test_deep_update_engine_inner_k_loops_do_not_spill(kernel_asm):
    # Engine4<true, 32, 4> (the update launches of chains of matrices with
    # m <= 4096): K step 32 = 2 sub-steps of 16 MFMAs. Its innermost K-step
    # loops must not spill. (The loop around them holds a scratch reload on
    # the path for tiles too short to claim a successor, K < 192, which no
    # plan takes: K is a multiple of 256.)
    loops = _k_step_loops(kernel_asm, r"phase_kernel4INS_7Engine4ILb1ELi32ELi4EEE", 32, innermost=True)
    kernels = {k for k, _, _, _ in loops}
    assert len(kernels) == 3, f"expected the update and last-update kernels (bf16 and fp32 W), found {kernels}"
    bad = [(k[-40:], n, s) for k, n, _, s in loops if s]
    assert not bad, f"K-step loops with scratch accesses (kernel, length, accesses): {bad}"
