"""Register and scratch use of the built conv kernels, read from the gfx950 code object's
metadata notes (no GPU needed).  A kernel that spills keeps per-lane scratch in memory
and runs far slower than its configuration was measured at, with the same results, so
no parity test notices; this test does.  Only the forced-tile configurations the
automatic choice never takes may use scratch: the four-wave 256x256 streaming block
(tile 17), the pipelined 256x256 block (tile 4) and the four-channel-gather variants
of the 64x256 and 128x256 streaming blocks (the host moves the four-channel gather to
other blocks)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "integer_quantized_nn_amd", "_build", "qconv.o")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# name patterns of the kernels allowed to use scratch (forced tiles only)
ALLOWED = [
    re.compile(r"qconv_streamINS0_9StreamCfgILi256ELi256ELi2ELi4ELi0ELi64ELi4EEE"),   # tile 17
    re.compile(r"qconv_pipeINS0_7PipeCfgILi256ELi256ELi2ELi4EEE"),                    # tile 4
    # four-channel gather (third flag after the configuration: C4 = true)
    re.compile(r"qconv_streamINS0_9StreamCfgILi64ELi256ELi1ELi3ELi0ELi64ELi4EEELb.ELb.ELb1E"),
    re.compile(r"qconv_streamINS0_9StreamCfgILi128ELi256ELi2ELi3ELi0ELi64ELi4EEELb.ELb.ELb1E"),
]


def _kernel_metadata():
    """(name, private segment bytes, vgpr count) of every kernel in qconv.o's gfx950
    code object."""
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    if not os.path.exists(OBJ):
        pytest.skip("the HIP library is not built (run __graft_entry__.build())")
    work = os.path.join(ROOT, "integer_quantized_nn_amd", "_build", "resources")
    os.makedirs(work, exist_ok=True)
    try:
        fatbin = os.path.join(work, "fatbin.bin")
        code = os.path.join(work, "qconv_gfx950.co")
        subprocess.run([tools[0], "--dump-section=.hip_fatbin=" + fatbin, OBJ, os.path.join(work, "host.o")],
                       check=True, capture_output=True)
        subprocess.run([tools[1], "--unbundle", "--type=o", "--input=" + fatbin, "--targets=" + TARGET,
                        "--output=" + code], check=True, capture_output=True)
        notes = subprocess.run([tools[2], "--notes", code], check=True, capture_output=True, text=True).stdout
    finally:
        shutil.rmtree(work, ignore_errors=True)
    out = []
    # each kernel's metadata map lists .name, then .private_segment_fixed_size, ...,
    # .vgpr_count (keys in alphabetical order)
    for block in notes.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        vgpr = re.search(r"\.vgpr_count:\s+(\d+)", block)
        if name and priv and vgpr:
            out.append((name.group(1), int(priv.group(1)), int(vgpr.group(1))))
    return out


def test_only_forced_tile_kernels_use_scratch():
    meta = _kernel_metadata()
    names = [m[0] for m in meta]
    assert len(meta) > 200, "kernel metadata not parsed (%d entries)" % len(meta)
    # the kernels of the benchmarked trunk are among them
    for must in ("qconv_stem_pool", "qconv_direct3x3", "qconv_pair", "qconv_stream"):
        assert any(must in n for n in names), must
    spilling = [(n, p) for n, p, _ in meta if p > 0]
    unexpected = [(n, p) for n, p in spilling if not any(a.search(n) for a in ALLOWED)]
    assert not unexpected, "kernels with scratch outside the forced-tile set:\n" + "\n".join(
        "%6d B  %s" % (p, n) for n, p in unexpected)


def test_no_kernel_exceeds_the_register_file():
    """At most 512 registers (VGPRs and AGPRs) per lane, the wave's whole file."""
    for n, _, v in _kernel_metadata():
        assert v <= 512, (n, v)
