"""The Dykstra cycle's hot block at M = 32 has no VALU instruction whose
three VGPR operands sit in one register bank.

A VGPR's bank is its number mod 4.  On gfx950 an instruction that reads
three operands from one bank issues at 0.57x the rate of one whose operands
are spread (a v_fmac_f32 loop, measured: two operands in one bank cost
nothing).  The compiler's register allocator does not model this, so a
change anywhere in the cycle loop can put the column updates' v_fmac
(total, E, row factor) into one bank; at 11-13 such instructions per cycle
the 16:32 launch ran 1-2% slower.  The kernel source picks a column order
for which the allocation has none; this test compiles the source as the
library is built and checks that it still has none.  The hot block is the
basic block holding the clamped products E = min(P V U, 1).  No GPU is used.
"""
import collections
import os
import re
import shutil

import pytest

from sparse_mask_search_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.hipcc()) is None
                                and not os.path.exists(build.hipcc()),
                                reason="hipcc is not installed")


def blocks(asm: str, symbol: str):
    """Instruction lists of the basic blocks of one kernel."""
    start = asm.index(symbol + ":")
    end = asm.index(".Lfunc_end", start)
    out, cur = [], []
    for line in asm[start:end].split("\n"):
        if line.startswith(".LBB") or line.startswith("; %bb"):
            out.append(cur)
            cur = []
        elif line.startswith("\t") and not line.strip().startswith((";", ".")):
            cur.append(line.strip())
    out.append(cur)
    return out


def vgpr_operands(ins: str):
    """First VGPR of each operand (None for SGPRs, constants, modifiers)."""
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    regs = []
    for p in parts[1].split(","):
        p = p.strip().split()[0] if p.strip() else ""
        m = re.match(r"^v(\d+)$", p) or re.match(r"^v\[(\d+):\d+\]$", p)
        regs.append(int(m.group(1)) if m else None)
    return parts[0], regs


def same_bank_triples(block):
    """VALU instructions reading >= 3 distinct VGPRs that all share a bank."""
    bad = []
    for ins in block:
        op, regs = vgpr_operands(ins)
        if not op.startswith("v_") or "_dpp" in op:
            continue
        srcs = {r for r in regs[1:] if r is not None}
        if op.startswith(("v_fmac", "v_mac")) and regs and regs[0] is not None:
            srcs.add(regs[0])  # the accumulator is read too
        if len(srcs) >= 3 and max(collections.Counter(r % 4 for r in srcs).values()) >= 3:
            bad.append(ins)
    return bad


def hot_block(asm: str, symbol: str):
    return max(blocks(asm, symbol), key=lambda b: sum("clamp" in i for i in b))


def test_checker_on_hand_written_blocks():
    assert same_bank_triples(["v_fmac_f32_e32 v40, v44, v48"]) == ["v_fmac_f32_e32 v40, v44, v48"]
    assert same_bank_triples(["v_fmac_f32_e32 v40, v45, v50"]) == []
    assert same_bank_triples(["v_fma_f32 v1, v4, v8, v12"]) == ["v_fma_f32 v1, v4, v8, v12"]
    assert same_bank_triples(["v_fma_f32 v4, v5, v8, v12"]) == []  # destination is not read
    assert same_bank_triples(["v_mul_f32_e64 v1, v4, v8 clamp"]) == []  # two sources
    assert same_bank_triples(["v_fmac_f32_e32 v4, v4, v8"]) == []  # two distinct registers
    assert same_bank_triples(["v_add_f32_dpp v4, v8, v12 quad_perm:[1,0,3,2]"]) == []
    assert same_bank_triples(["v_fmac_f32_e32 v40, s4, v48"]) == []


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("isa") / "tsenor_kernels.s")
    with open(build.device_asm("tsenor_kernels.hip", out)) as f:
        return f.read()


MASK32 = "_ZN6tsenor12_GLOBAL__N_111mask_kernelILi32ELb{bf}ELb0EEEvNS_6MatJobENS_6ParamsE"
BATCHED32 = "_ZN6tsenor12_GLOBAL__N_114batched_kernelILi32ELb{bf}ELb0EEEvPKNS_6MatJobEilNS_6ParamsE"


@pytest.mark.parametrize("symbol", [MASK32.format(bf=1), MASK32.format(bf=0),
                                    BATCHED32.format(bf=1), BATCHED32.format(bf=0)],
                         ids=["mask-bf16", "mask-f32", "batched-bf16", "batched-f32"])
def test_m32_hot_block_has_no_same_bank_triples(kernel_asm, symbol):
    hot = hot_block(kernel_asm, symbol)
    assert sum("clamp" in i for i in hot) == 128  # the 8 x 16 products of one lane's tile
    assert same_bank_triples(hot) == []
