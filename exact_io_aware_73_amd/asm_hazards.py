"""Check the device assembly of kernels that issue matrix products through
inline assembly.

The d = 128 kernels (the forward's rows64 pipeline, its split-KV form and the
backward's dK/dV kernel) keep some matrix-product accumulators in AGPRs by
writing those products as inline `v_mfma_*` statements.  The compiler does
not see such a statement as matrix-core work, so it does not wait out the
product's write latency before an instruction of its own touches the
accumulator (a register move it inserts, a vector-ALU read).  The kernels
wait themselves (`s_nop` after the products or before reading the
accumulators); this module checks, on the compiled assembly, that no other
instruction touches an AGPR written by such a product within `wait_states`
wait states along any control-flow path.

Wait states are counted conservatively: `s_nop k` gives k + 1, every other
instruction one.  A product that accumulates into the same AGPRs it read is
not a violation (dependent products into one accumulator need no wait).

    python -m exact_io_aware_73_amd.asm_hazards          # the three sources
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build as B

# sources whose kernels hold accumulators in AGPRs through inline products
SOURCES = ("attn_bwd.hip", "attn_fwd_bf16_rows64.hip", "attn_fwd_bf16_split.hip")
# the longest write latency a matrix product needs before another
# instruction may touch its result (16-pass products), with a margin
WAIT_STATES = 19

_AGPR_PRODUCT = re.compile(r"v_mfma\S*\s+a\[(\d+):(\d+)\]")
_BRANCH = ("s_branch", "s_cbranch", "s_endpgm", "s_setpc")


def device_asm(source: str) -> str:
    """Device assembly of csrc/<source>, compiled with the library's flags."""
    flags = [f for f in B.CFLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    flags += B.FILE_FLAGS.get(source, [])
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        B._run([B.HIPCC, *flags, "-S", "--cuda-device-only", os.path.join(B.CSRC, source), "-o", out])
        with open(out) as f:
            return f.read()


def _agprs(ins: str) -> set[int]:
    regs = {int(a) for a in re.findall(r"\ba(\d+)\b", ins)}
    for lo, hi in re.findall(r"\ba\[(\d+):(\d+)\]", ins):
        regs |= set(range(int(lo), int(hi) + 1))
    return regs


def _states(ins: str) -> int:
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


def _blocks(body: list[str]):
    """Basic blocks (label, instructions) and their successors."""
    blocks, cur = [], {"label": None, "ins": []}
    for line in body:
        if re.match(r"\.LBB\S+:$", line):
            blocks.append(cur)
            cur = {"label": line[:-1], "ins": []}
            continue
        cur["ins"].append(line)
        if line.startswith(_BRANCH):
            blocks.append(cur)
            cur = {"label": None, "ins": []}
    blocks.append(cur)
    blocks = [b for b in blocks if b["ins"] or b["label"]]
    index = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    succ = []
    for i, b in enumerate(blocks):
        last = b["ins"][-1] if b["ins"] else ""
        s = []
        m = re.match(r"s_c?branch\S*\s+(\.LBB\S+)", last)
        if m and m.group(1) in index:
            s.append(index[m.group(1)])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def agpr_hazards(asm: str, wait_states: int = WAIT_STATES, max_blocks: int = 8) -> dict[str, list]:
    """{kernel: [(block label, instruction), ...]} for every instruction that
    touches an AGPR an inline matrix product wrote fewer than `wait_states`
    wait states earlier, following up to `max_blocks` blocks per path.
    Kernels without AGPR-accumulating products are left out."""
    result = {}
    for m in re.finditer(r"^([A-Za-z_][A-Za-z0-9_]*):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        if end < 0:
            continue
        body = []
        for raw in asm[m.end():end].splitlines()[1:]:
            line = raw.split(";")[0].strip()
            if line and (not line.startswith(".") or re.match(r"\.LBB\S+:$", line)):
                body.append(line)
        if not any(_AGPR_PRODUCT.match(l) for l in body):
            continue
        blocks, succ = _blocks(body)
        bad = []

        def walk(bi, pending, start, depth):
            for ins in blocks[bi]["ins"][start:]:
                if not pending:
                    return
                regs = _agprs(ins)
                pm = _AGPR_PRODUCT.match(ins)
                if pm:   # a product reading or writing other pending AGPRs
                    own = set(range(int(pm.group(1)), int(pm.group(2)) + 1))
                    if (regs - own) & pending.keys():
                        bad.append((blocks[bi]["label"], ins))
                elif regs & pending.keys():
                    bad.append((blocks[bi]["label"], ins))
                    return
                k = _states(ins)
                pending = {r: v - k for r, v in pending.items() if v - k > 0}
            if pending and depth < max_blocks:
                for s in succ[bi]:
                    walk(s, dict(pending), 0, depth + 1)

        for bi, b in enumerate(blocks):
            for j, ins in enumerate(b["ins"]):
                pm = _AGPR_PRODUCT.match(ins)
                if pm:
                    walk(bi, {r: wait_states for r in range(int(pm.group(1)), int(pm.group(2)) + 1)}, j + 1, 0)
        result[m.group(1)] = bad
    return result


def main(argv):
    failed = False
    for src in argv or SOURCES:
        for kernel, bad in agpr_hazards(device_asm(src)).items():
            print(f"{src}: {kernel}: {len(bad)} violation(s)")
            for label, ins in bad[:5]:
                print(f"    {label}: {ins}")
            failed |= bool(bad)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
