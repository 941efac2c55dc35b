"""Properties of the generated gfx950 code that the kernels' correctness relies on.

The dK/dV kernel of the backward pass issues its matrix products as inline
assembly with fixed register classes (K, V, dK, dV in accumulation registers, S
and dP in vector registers) and inserts the wait states around them itself,
because the compiler's hazard checks do not see an MFMA inside an asm statement.
That is sound only while the compiler neither spills nor moves those registers
inside the tile loop: a copy or spill placed right after such a product would
read its result before the product has finished. These tests compile the kernel
to assembly (CPU only; hipcc cross-compiles) and check that every basic block
holding matrix products is free of register-file moves and scratch accesses.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from exact_attention_flash_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _assembly(source: str) -> str:
    try:
        hipcc = build.hipcc_path()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", *build.DEVICE_FLAGS,
               f"-I{os.path.join(ROOT, 'include')}", "--cuda-device-only", "-S", "-o", out, source]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert res.returncode == 0, res.stdout[-2000:]
        with open(out) as f:
            return f.read()


def _blocks(asm: str, kernel: str):
    m = re.search(r"^" + re.escape(kernel) + r":(.*?)s_endpgm", asm, re.S | re.M)
    assert m, kernel
    blocks, name, lines = [], "entry", []
    for ln in m.group(1).split("\n"):
        mm = re.match(r"^(\.LBB\S+):", ln)
        if mm:
            blocks.append((name, lines))
            name, lines = mm.group(1), []
            continue
        t = ln.strip()
        if t and not t.startswith(";"):
            lines.append(t.split()[0])
    blocks.append((name, lines))
    return blocks


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_dkdv_product_blocks_have_no_moves_or_spills():
    asm = _assembly(os.path.join(ROOT, "exact_attention_flash_amd", "csrc", "bwd_kernel.hip"))
    kernels = re.findall(r"^(_ZN2fa3bwd8bwd_dkdv\S+):", asm, re.M)
    assert len(kernels) == 8  # {bf16, fp16} x {64, 128} x {causal, not}
    for k in kernels:
        for name, ins in _blocks(asm, k):
            if not any("mfma" in i for i in ins):
                continue
            moves = [i for i in ins if "accvgpr" in i or i.startswith("scratch_")]
            assert not moves, f"{k} block {name}: {len(moves)} register moves/spills beside asm products"
