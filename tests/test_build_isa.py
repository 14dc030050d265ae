"""Build checks on the gfx950 code of the ring kernel (CPU only: hipcc cross-compiles).

The kernel reads its launch arguments through the kernarg-segment pointer, which is
only valid in the kernel's own body: a function the compiler leaves out of line would
see a null base. The kernel therefore evaluates the pointer once and passes it down,
and these checks pin that no other function is called from the kernels except the
trace hook (which takes the pointer as an argument).
"""

import os
import re
import tempfile

from overlap_attention_amd import build as mkbuild


def _asm():
    with tempfile.TemporaryDirectory() as d:
        return mkbuild.device_asm(os.path.join(d, "k.s"))


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
