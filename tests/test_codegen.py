"""Code generation checks on the gfx950 assembly of the GEMM kernels (CPU only:
hipcc cross-compiles).

A buffer load whose descriptor the compiler cannot prove uniform is wrapped
in a loop over the lanes' distinct descriptors (v_readfirstlane, compare,
exec mask, load, s_cbranch_execnz back-edge).  Every descriptor here is built
from kernel arguments, so such a loop is never needed, and where it appeared
it put each weight load behind a branch and slowed the kernels (one layout of
the argument struct cost the gate/value projection 17 %).  This test fails if
any GEMM kernel contains one.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from groupwise_int_weight_amd import build

    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "ngq_gemm.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    src = os.path.join(build.CSRC, "ngq_gemm.hip")
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", out], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def kernels(asm):
    for m in re.finditer(r"^(_ZN3ngq3dev\d+(gemm\w*?kernel)\S*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].splitlines()


def waterfall_blocks(lines):
    labels = [k for k, ln in enumerate(lines) if re.match(r"^\.LBB\d+_\d+:", ln)]
    n = 0
    for a, b in zip([0] + labels, labels + [len(lines)]):
        ops = [ln.split()[0] for ln in (t.strip() for t in lines[a:b]) if ln and not ln.startswith((";", "."))]
        if any(o.startswith("buffer_load") for o in ops) and "v_readfirstlane_b32" in ops \
                and "s_cbranch_execnz" in ops:
            n += 1
    return n


def test_every_gemm_kernel_is_present(asm):
    found = {re.match(r"_ZN3ngq3dev\d+(gemm\w*?kernel)", k).group(1) for k, _ in kernels(asm)}
    for fam in ("gemm_xres_kernel", "gemm_kernel", "gemm_multi_kernel", "gemm_splitk_kernel", "gemm_wide_kernel",
                "gemm_tiled_kernel", "gemm_tiled_sx_kernel", "gemm_stream_kernel", "gemm_dot_kernel",
                "gemm_multi_dot_kernel", "gemm_multi_stream_kernel"):
        assert fam in found, (fam, sorted(found))


def test_no_load_waits_on_a_descriptor_loop(asm):
    bad = {name: n for name, lines in kernels(asm) if (n := waterfall_blocks(lines))}
    assert not bad, bad


def test_decode_kernels_use_no_scratch(asm):
    """The streaming, VALU-step, split-K and one-tile-per-workgroup fused kernels keep
    everything in registers: no spills, and no private copy of the argument
    block (the fused kernels index their projection descriptors with a
    workgroup-uniform value)."""
    meta = {}
    for m in re.finditer(r"\.name:\s+(_ZN3ngq3dev\d+(gemm_(?:multi_dot|multi_stream|stream|dot|splitk)_kernel)\S*)",
                         asm):
        start = asm.rfind("\n  - ", 0, m.start())
        end = asm.find("\n  - ", m.end())
        block = asm[start:end if end > 0 else len(asm)]
        fields = dict(re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count):\s+(\d+)", block))
        meta[m.group(1)] = fields
    assert {re.match(r"_ZN3ngq3dev\d+(\w+?kernel)", k).group(1) for k in meta} == {
        "gemm_multi_dot_kernel", "gemm_multi_stream_kernel", "gemm_stream_kernel", "gemm_dot_kernel",
        "gemm_splitk_kernel"}
    bad = {k: v for k, v in meta.items() if v.get("private_segment_fixed_size") != "0" or v.get("vgpr_spill_count") != "0"}
    assert not bad, bad
