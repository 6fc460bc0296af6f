"""Properties of the compiled gfx950 code that the pipelined GEMM tiles rely
on, checked on the device assembly of csrc/grouped_gemm.hip (host-only:
hipcc cross-compiles, no GPU needed).

The ping-pong tiles let a tile's first three stage waits skip the previous
epilogue's stores by counting them: every wave must issue exactly STORES
stores per epilogue, also where several go to the same dropped offset (the
compiler would otherwise merge or remove those), and no store may sit in a
loop over lanes (a resource the compiler cannot prove uniform)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_steered_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                  else None)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gg.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "grouped_gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def kernel_body(asm, pattern):
    """The assembly of the one kernel whose mangled name matches pattern."""
    heads = [m for m in re.finditer(r"^(_Z\S+):", asm, re.M) if re.search(pattern, m.group(1))]
    assert len(heads) == 1, f"{pattern}: {len(heads)} kernels"
    start = heads[0].end()
    end = asm.index(".Lfunc_end", start)
    return asm[start:end]


# (kernel: PipeShape<256, BN, GATEUP, 32, 8, 2, PACKED, HBLK> with gate_up
# Lb1E or down Lb0E, then the weight layout and the h layout, each Lb0E rows
# / Lb1E blocked; STORES, epilogue copies).  bf16 ping-pong: full tile,
# half-height tile, and the stand-in before the first tile; W4A16
# ping-pong: the same in gate_up, no half-height tile in down
CASES = [(rf"17grouped_pp_kernel.*{proj}ELi32ELi8ELi2E{w}E{h}E", stores, 3)
         for proj, stores in (("Lb1", 16), ("Lb0", 32))
         for w in ("Lb0", "Lb1") for h in ("Lb0", "Lb1")] + [
    (r"20grouped_pp_w4_kernel.*Lb1ELi32", 16, 3),
    (r"20grouped_pp_w4_kernel.*Lb0ELi32", 32, 2),
]


@pytest.mark.parametrize("pattern,stores,copies", CASES)
def test_epilogue_store_count(asm, pattern, stores, copies):
    body = kernel_body(asm, pattern)
    n = len(re.findall(r"^\s*buffer_store_dwordx[24]\b", body, re.M))
    assert n == stores * copies, f"{n} epilogue stores, expected {copies} x {stores}"


@pytest.mark.parametrize("pattern,stores,copies", CASES)
def test_no_store_in_lane_loop(asm, pattern, stores, copies):
    body = kernel_body(asm, pattern).splitlines()
    for i, line in enumerate(body):
        if re.match(r"^\s*buffer_store_dwordx[24]\b", line):
            before = "\n".join(body[max(0, i - 4):i])
            assert "saveexec" not in before, f"store in a loop over lanes:\n{before}\n{line}"
