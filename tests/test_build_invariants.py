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

The direct-to-LDS loads are inline assembly too, and read scalar registers (the
buffer descriptor, M0) that a VALU instruction may have written just before; the
hazard audit below checks the required wait states around every such load and
every matrix product in the forward, backward and FP8 kernels (it flags the code
generated before the loads carried their own wait states).
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


# ---- wait states around instructions the compiler cannot see inside inline asm ----
# gfx950 needs software wait states between a VALU write of a register and some
# later readers, and after an MFMA before a VALU access of its result. The compiler
# inserts them for its own instructions; for asm statements the kernels insert them
# themselves. The checks below walk the generated code in program order inside
# each basic block, counting one wait state per instruction and k + 1 for s_nop k.

_REG = re.compile(r"\b([vas])\[(\d+):(\d+)\]|\b([vas])(\d+)\b")


def _regs(text: str):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _function(asm: str, kernel: str):
    m = re.search(r"^" + re.escape(kernel) + r":(.*?)s_endpgm", asm, re.S | re.M)
    assert m, kernel
    blocks, cur = [], []
    for ln in m.group(1).split("\n"):
        if re.match(r"^\.LBB\S+:", ln):
            blocks.append(cur)
            cur = []
            continue
        t = ln.split(";")[0].strip()
        if t and not t.startswith("."):
            cur.append(t)
    blocks.append(cur)
    return blocks


def _waits(ins: str) -> int:
    if ins.startswith("s_nop"):
        return int(ins.split()[1], 0) + 1
    return 1


def _operands(ins: str):
    parts = ins.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def _is_valu(op: str) -> bool:
    return op.startswith("v_") and "mfma" not in op


def _hazards(asm: str, kernel: str):
    """Violations in one kernel: LDS-DMA loads without five wait states after a VALU
    write of an SGPR they read; MFMAs without two after a VALU write of a source;
    VALU accesses of an MFMA result within twelve wait states of the MFMA."""
    bad = []
    for blk in _function(asm, kernel):
        for n, ins in enumerate(blk):
            op = ins.split()[0]
            ops = _operands(ins)
            if op.startswith("buffer_load") and ins.endswith("lds"):
                reads = _regs(",".join(ops[1:]))
                w = 0
                for prev in reversed(blk[:n]):
                    if w >= 5:
                        break
                    pop = prev.split()[0]
                    if _is_valu(pop) and _regs(_operands(prev)[0]) & reads:
                        bad.append(f"{kernel}: '{prev}' then '{ins}' within {w} wait states")
                    w += _waits(prev)
                if w < 5:  # the window reaches a block start: the predecessor is unknown
                    bad.append(f"{kernel}: '{ins}' only {w} wait states into its block")
            elif "mfma" in op:
                srcs = _regs(",".join(ops[1:3]))
                w = 0
                for prev in reversed(blk[:n]):
                    if w >= 2:
                        break
                    pop = prev.split()[0]
                    if (_is_valu(pop) or pop.startswith("v_accvgpr_write")) and _regs(_operands(prev)[0]) & srcs:
                        bad.append(f"{kernel}: '{prev}' then '{ins}' within {w} wait states")
                    w += _waits(prev)
                dst = _regs(ops[0])
                w = 0
                for nxt in blk[n + 1:]:
                    if w >= 12:
                        break
                    nop = nxt.split()[0]
                    if _is_valu(nop) and _regs(",".join(_operands(nxt))) & dst:
                        bad.append(f"{kernel}: '{ins}' then '{nxt}' within {w} wait states")
                    w += _waits(nxt)
    return bad


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("source", ["fwd_kernel.hip", "fwd_sp.hip", "bwd_kernel.hip", "fwd_fp8.hip"])
def test_inline_asm_wait_states(source):
    asm = _assembly(os.path.join(ROOT, "exact_attention_flash_amd", "csrc", source))
    kernels = re.findall(r"^(_Z\S+):\s*(?:;|$)", asm, re.M)
    assert kernels
    lds_loads = 0
    bad = []
    for k in kernels:
        bad += _hazards(asm, k)
        lds_loads += sum(1 for blk in _function(asm, k) for i in blk if i.startswith("buffer_load") and i.endswith("lds"))
    assert lds_loads > 0
    assert not bad, "\n".join(bad[:20]) + f"\n({len(bad)} in all)"
