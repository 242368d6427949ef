"""Build-time check of the gfx950 assembly of the library's own kernels.

A vector-memory store of more than 64 bits (buffer_store_dwordx3/x4, global_store_b128
...) reads its data registers after it issues, and the hardware needs one wait state
before an instruction may overwrite them.  The compiler inserts that wait state, except
for buffer stores whose scalar offset field is a register: it assumes the hazard away
there.  On MI355X such code stored the new register contents (an integer from the next
address computation) instead of the data, in the first dword of some lanes.  The kernels
therefore pass the whole store offset in the vector operand (scalar offset 0); build.py
compiles every kernel source to assembly and refuses the library if any wide store is
directly followed by a write of its data registers.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"v\[(\d+):(\d+)\]")
_ONE = re.compile(r"v(\d+)")
_WIDE_STORE = re.compile(r"^(buffer_store_dword(x3|x4)|buffer_store_b(96|128)|"
                         r"global_store_dword(x3|x4)|global_store_b(96|128)|"
                         r"flat_store_dword(x3|x4)|flat_store_b(96|128))\b")


def _vregs(tok: str) -> set:
    tok = tok.strip()
    m = _RANGE.fullmatch(tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _ONE.fullmatch(tok)
    return {int(m.group(1))} if m else set()


def _store_data(ins: str) -> set:
    ops = ins.split(None, 1)[1].split(",")
    # buffer_store vdata, vaddr, srsrc, soffset; global/flat_store vaddr, vdata, ...
    return _vregs(ops[0] if ins.startswith("buffer_") else ops[1])


def _dest(ins: str) -> set:
    parts = ins.split(None, 1)
    if len(parts) < 2 or parts[0].startswith(("s_", "buffer_store", "global_store",
                                              "flat_store", "ds_write", "ds_store")):
        return set()
    return _vregs(parts[1].split(",")[0])


def store_data_overwrites(asm: str) -> list:
    """[(kernel, store, writer)] for every store of more than 64 bits whose data
    registers are written by the next instruction with no wait state in between
    (labels and conditional branches are followed through to the fall-through code)."""
    found = []
    for fm in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", fm.end())
        body = asm[fm.end():end if end >= 0 else len(asm)]
        ins = [l.split(";")[0].strip() for l in body.splitlines()]
        ins = [l for l in ins if l and not (l.startswith(".") and not l.startswith(".LBB"))]
        for i, t in enumerate(ins):
            if not _WIDE_STORE.match(t):
                continue
            data = _store_data(t)
            for nxt in ins[i + 1:]:
                if nxt.endswith(":"):
                    continue  # a label costs nothing; keep looking at the fall-through
                if nxt.startswith(("s_nop", "s_cbranch", "s_waitcnt")):
                    break  # at least one wait state before anything else issues
                if nxt.startswith(("s_branch", "s_endpgm", "s_setpc")):
                    break
                if _dest(nxt) & data:
                    found.append((fm.group(1).rstrip(":"), t, nxt))
                break
    return found
