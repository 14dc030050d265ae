"""Build checks on the gfx950 code of the kernels (CPU only: hipcc cross-compiles).

- The ring kernel reads its launch arguments through the kernarg-segment pointer,
  which is only valid in the kernel's own body: a function the compiler leaves out of
  line would see a null base. The kernel therefore evaluates the pointer once and
  passes it down, and these checks pin that no other function is called from the
  kernels except the trace hook (which takes the pointer as an argument).
- The block copies (global_load_lds_dwordx4) are inline asm with an SGPR base. A
  memory instruction that reads an SGPR written by a vector instruction (v_readlane,
  v_readfirstlane, a compare) needs 5 wait states in between, which the compiler does
  not insert for inline asm operands; a build in which a spill reload landed right
  before a copy read a stale base and faulted. Every copy must therefore sit at least
  5 wait states after any vector write of its base, whatever the register allocation.
"""

import os
import re
import tempfile

import pytest

from overlap_attention_amd import build as mkbuild


def _asm(source=mkbuild.SOURCES[0]):
    with tempfile.TemporaryDirectory() as d:
        return mkbuild.device_asm(os.path.join(d, "k.s"), source)


def test_only_trace_hook_is_called_out_of_line():
    s = _asm()
    functions = set(re.findall(r"^\s*\.type\s+(\S+),@function", s, re.M))
    kernels = set(re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", s, re.M))
    assert len([k for k in kernels if "ring_attn_kernel" in k]) == 2, kernels  # D = 64 and D = 128
    others = functions - kernels
    assert all("trace_rec" in f for f in others), others
    # Every call goes to the trace hook: each s_swappc takes an address formed from a
    # pc-relative relocation, and every such relocation names the hook.
    calls = len(re.findall(r"\bs_swappc_b64\b", s))
    targets = re.findall(r"(\S+)@rel32@lo", s)
    assert calls > 0 and len(targets) == calls, (calls, targets)
    assert all("trace_rec" in t for t in targets), set(targets)


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def copy_base_hazards(asm):
    """(copies, list of copies whose SGPR base a vector instruction writes fewer than 5
    wait states before). Wait states are counted as issued instructions, s_nop N as
    N + 1; the search stops at a label or a branch (a path from elsewhere begins)."""
    lines = [l.strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith((";", "."))]
    copies, bad = 0, []
    for i, l in enumerate(lines):
        if not l.startswith("global_load_lds"):
            continue
        copies += 1
        base = _sgprs(l.split(",")[1].strip())
        assert base, l
        ws = 0
        for p in reversed(lines[max(0, i - 16):i]):
            op = p.split()[0]
            if p.endswith(":") or op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_swappc")):
                if ws < 5:
                    bad.append((l, "path joins here " + p))
                break
            if op == "s_nop":
                ws += int(p.split()[1], 0) + 1
            else:
                if op.startswith("v_") and _sgprs(p.split()[1].rstrip(",")) & base:
                    bad.append((l, p))
                    break
                ws += 1
            if ws >= 5:
                break
    return copies, bad


@pytest.mark.parametrize("source", [mkbuild.SOURCES[0], mkbuild.SOURCES[2]], ids=["ring", "allgather_gemm"])
def test_block_copies_wait_after_vector_writes_of_their_base(source):
    copies, bad = copy_base_hazards(_asm(source))
    assert copies > 0
    assert not bad, bad[:5]


def test_hazard_check_flags_a_reload_right_before_a_copy():
    asm = """
    v_readlane_b32 s2, v254, 22
    s_add_i32 m0, s0, 0x8000
    v_readlane_b32 s3, v254, 23
    global_load_lds_dwordx4 v153, s[2:3]
    s_nop 4
    global_load_lds_dwordx4 v152, s[2:3]
    """
    copies, bad = copy_base_hazards(asm)
    assert copies == 2 and len(bad) == 1 and "v_readlane_b32 s3" in bad[0][1]
