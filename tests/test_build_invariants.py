"""Properties of the generated gfx950 code that the kernels' correctness relies on.

The dK/dV and dQ kernels of the backward pass issue their matrix products as
inline assembly with fixed register classes (K, V, dK, dV, or Q, dO, dQ in
accumulation registers; S and dP in vector registers) and insert the wait states
around them themselves,
because the compiler's hazard checks do not see an MFMA inside an asm statement.
That is sound only while the compiler neither spills nor moves those registers
inside the tile loop: a copy or spill placed right after such a product would
read its result before the product has finished. These tests compile the kernel
to assembly (CPU only; hipcc cross-compiles) and check that no register-file
move or scratch access sits between two matrix products of a basic block.

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
def test_backward_product_blocks_have_no_moves_or_spills():
    asm = _assembly(os.path.join(ROOT, "exact_attention_flash_amd", "csrc", "bwd_kernel.hip"))
    kernels = re.findall(r"^(_ZN2fa3bwd(?:8bwd_dkdv|6bwd_dq)\S+):", asm, re.M)
    assert len(kernels) == 16  # {dK/dV, dQ} x {bf16, fp16} x {64, 128} x {causal, not}
    for k in kernels:
        for name, ins in _blocks(asm, k):
            at = [n for n, i in enumerate(ins) if "mfma" in i]
            if not at:
                continue
            # set-up before the block's first product (K and V into the accumulation
            # registers, dK and dV zeroed) and the read-out after its last one (after
            # the drain) are allowed; the wait-state audit below checks those moves
            # as VALU accesses like any other
            moves = [i for i in ins[at[0]:at[-1]] if "accvgpr" in i or i.startswith("scratch_")]
            assert not moves, f"{k} block {name}: {len(moves)} register moves/spills between asm products"


# ---- wait states around instructions the compiler cannot see inside inline asm ----
# gfx950 needs software wait states between a VALU write of a register and some
# later readers, and after an MFMA before a VALU access of its result. The compiler
# inserts them for its own instructions; for asm statements the kernels insert them
# themselves. The checks below walk the generated code in program order inside
# each basic block, counting one wait state per instruction and k + 1 for s_nop k.

_REG = re.compile(r"\b([vas])\[(\d+):(\d+)\]|\b([vas])(\d+)\b|\b(m0)\b")
_M0 = ("m", 0)


def _regs(text: str):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        elif m.group(6):
            out.add(_M0)
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


_LABEL = re.compile(r"^(\.L[\w$.]+):")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.L[\w$.]+)")


def _function(asm: str, kernel: str):
    """The kernel's code as basic blocks with their control-flow edges. Every label
    starts a block (the compiler's and those of asm statements that branch inside
    themselves); a block ends at a label or after a branch. Returns (blocks, succ,
    pred): instruction lists and successor / predecessor block indices."""
    m = re.search(r"^" + re.escape(kernel) + r":(.*?)^\.Lfunc_end", asm, re.S | re.M)
    assert m, kernel
    blocks, labels, cur, cur_label = [], {}, [], None

    def close():
        labels.setdefault(cur_label, len(blocks)) if cur_label else None
        blocks.append(cur)

    for ln in m.group(1).split("\n"):
        lm = _LABEL.match(ln.strip())
        if lm:
            close()
            cur, cur_label = [], lm.group(1)
            continue
        t = ln.split(";")[0].strip()
        if t and not t.startswith("."):
            cur.append(t)
            if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
                close()
                cur, cur_label = [], None
    close()
    succ = [[] for _ in blocks]
    for i, blk in enumerate(blocks):
        last = blk[-1] if blk else ""
        bm = _BRANCH.match(last)
        if bm:
            assert bm.group(2) in labels, f"{kernel}: branch to unknown label {bm.group(2)}"
            succ[i].append(labels[bm.group(2)])
        if not last.startswith(("s_branch ", "s_setpc", "s_endpgm")) and i + 1 < len(blocks):
            succ[i].append(i + 1)
    pred = [[] for _ in blocks]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return blocks, succ, pred


def _waits(ins: str) -> int:
    if ins.startswith("s_nop"):
        return int(ins.split()[1], 0) + 1
    return 1


def _operands(ins: str):
    parts = ins.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def _is_valu(op: str) -> bool:
    return op.startswith("v_") and "mfma" not in op


def _window(cfg, b, n, need, backward):
    """Every instruction within `need` wait states before (after) instruction n of
    block b, on every path through the control-flow graph, with the wait states
    between: a list of (instruction, wait states). A window that reaches the start of
    the kernel ends there (nothing ran before it)."""
    blocks, succ, pred = cfg
    out, seen = [], set()
    stack = [(b, n, 0)]
    while stack:
        b, n, w = stack.pop()
        blk = blocks[b]
        seq = reversed(blk[:n]) if backward else blk[n + 1:]
        for ins in seq:
            if w >= need:
                break
            out.append((ins, w))
            w += _waits(ins)
        else:
            for nb in (pred[b] if backward else succ[b]):
                key = (nb, w)
                if key not in seen:
                    seen.add(key)
                    stack.append((nb, len(blocks[nb]) if backward else -1, w))
    return out


def _hazards(asm: str, kernel: str):
    """Violations in one kernel, on every control-flow path: LDS-DMA loads without
    five wait states after a VALU write of an SGPR they read; MFMAs without two after
    a VALU write of a source; VALU accesses of an MFMA result within twelve wait
    states of the MFMA."""
    bad = []
    cfg = _function(asm, kernel)
    for b, blk in enumerate(cfg[0]):
        for n, ins in enumerate(blk):
            op = ins.split()[0]
            ops = _operands(ins)
            if op.startswith("buffer_load") and ins.endswith("lds"):
                # the descriptor and soffset, and M0 (the LDS address, an implicit operand)
                reads = _regs(",".join(ops[1:])) | {_M0}
                for prev, w in _window(cfg, b, n, 5, True):
                    pop = prev.split()[0]
                    written = _regs(_operands(prev)[0]) if _operands(prev) else set()
                    if _is_valu(pop) and written & reads:
                        bad.append(f"{kernel}: '{prev}' then '{ins}' within {w} wait states")
                    elif pop.startswith("s_") and _M0 in written and w < 1:
                        bad.append(f"{kernel}: '{prev}' then '{ins}' with no wait state after the M0 write")
            elif "mfma" in op:
                srcs = _regs(",".join(ops[1:3]))
                for prev, w in _window(cfg, b, n, 2, True):
                    pop = prev.split()[0]
                    if (_is_valu(pop) or pop.startswith("v_accvgpr_write")) and _regs(_operands(prev)[0]) & srcs:
                        bad.append(f"{kernel}: '{prev}' then '{ins}' within {w} wait states")
                dst = _regs(ops[0])
                for nxt, w in _window(cfg, b, n, 12, False):
                    if _is_valu(nxt.split()[0]) and _regs(",".join(_operands(nxt))) & dst:
                        bad.append(f"{kernel}: '{ins}' then '{nxt}' within {w} wait states")
    return bad


def test_hazard_windows_follow_control_flow():
    """The audit follows a window across branches: a VALU read of an MFMA result in
    the block a branch leads to, or a VALU write of a load's descriptor at the end of
    a predecessor, is found (synthetic listings, no compiler needed)."""
    fwd = "\n".join(["_k:", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
                       "s_cbranch_scc1 .LBB0_2", "s_nop 15", ".LBB0_2:", "v_add_f32 v30, v3, v4", "s_endpgm", ".Lfunc_end0:"])
    assert any("v_add_f32 v30, v3, v4" in x for x in _hazards(fwd, "_k"))
    fine = fwd.replace("s_cbranch_scc1 .LBB0_2", "s_nop 11\ns_cbranch_scc1 .LBB0_2")
    assert not _hazards(fine, "_k")
    back = "\n".join(["_k:", "v_readfirstlane_b32 s4, v1", "s_branch .LBB0_1", ".LBB0_1:",
                       "buffer_load_dwordx4 v2, s[4:7], 0 offen lds", "s_endpgm", ".Lfunc_end0:"])
    assert any("v_readfirstlane_b32 s4" in x for x in _hazards(back, "_k"))
    loop = "\n".join(["_k:", "s_nop 7", ".LBB0_1:", "buffer_load_dwordx4 v2, s[4:7], 0 offen lds",
                       "v_readfirstlane_b32 s4, v1", "s_cbranch_scc1 .LBB0_1", "s_endpgm", ".Lfunc_end0:"])
    assert any("v_readfirstlane_b32 s4" in x for x in _hazards(loop, "_k"))
    # M0 is read by every load to LDS: five wait states after a VALU write, one after a scalar one
    m0 = ["_k:", "s_nop 7", "s_mov_b32 m0, s9", "buffer_load_dwordx4 v2, s[4:7], 0 offen lds", "s_endpgm",
          ".Lfunc_end0:"]
    assert any("s_mov_b32 m0" in x for x in _hazards("\n".join(m0), "_k"))
    assert not _hazards("\n".join(m0[:3] + ["s_nop 0"] + m0[3:]), "_k")
    m0v = ["_k:", "s_nop 7", "v_readfirstlane_b32 m0, v3", "s_nop 3", "buffer_load_dwordx4 v2, s[4:7], 0 offen lds",
           "s_endpgm", ".Lfunc_end0:"]
    assert any("v_readfirstlane_b32 m0" in x for x in _hazards("\n".join(m0v), "_k"))


def test_uniform_addresses_are_not_sign_extended():
    """readfirstlane yields an int: widening it straight into a 64-bit address
    sign-extends a low half with bit 31 set over the high half (an unmapped
    address). Every address made wave-uniform goes through 32-bit unsigned halves."""
    csrc = os.path.join(ROOT, "exact_attention_flash_amd", "csrc")
    pat = re.compile(r"(\(\s*u?int64_t\s*\)|static_cast<\s*u?int64_t\s*>\(|\|)\s*__builtin_amdgcn_readfirstlane")
    bad = []
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            text = re.sub(r"\s+", " ", open(os.path.join(csrc, f)).read())
            bad += [f"{f}: ...{text[max(0, m.start() - 60):m.end() + 20]}..." for m in pat.finditer(text)]
    assert not bad, "\n".join(bad)
    bad_src = "x = ((uint64_t)__builtin_amdgcn_readfirstlane(hi) << 32) | __builtin_amdgcn_readfirstlane(lo);"
    assert pat.search(bad_src)


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
        lds_loads += sum(1 for blk in _function(asm, k)[0] for i in blk if i.startswith("buffer_load") and i.endswith("lds"))
    assert lds_loads > 0
    assert not bad, "\n".join(bad[:20]) + f"\n({len(bad)} in all)"


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("source", ["fwd_kernel.hip", "fwd_sp.hip", "bwd_kernel.hip", "fwd_fp8.hip"])
def test_no_fused_dot2(source):
    """No kernel may contain v_dot2*: the compiler once fused the fp16 widening and
    FMAs of the dQ kernel's D = rowsum(dO ∘ O) into v_dot2c_f32_f16 and issued the
    first pair's operands for all four pairs of a 16-byte vector, so D held a quarter
    of the sum four times. The kernels keep such sums as widened FMAs."""
    asm = _assembly(os.path.join(ROOT, "exact_attention_flash_amd", "csrc", source))
    dots = sorted({ln.split()[0] for ln in asm.split("\n") if ln.strip().startswith("v_dot2")})
    assert not dots, f"{source}: {dots}"
