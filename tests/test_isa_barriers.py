"""The built library's own gfx950 code, disassembled: no kernel has two workgroup barriers with
nothing between them but waits.

Such a pair is what remains when the compiler moves the LDS reads of a staged tile from between
two __syncthreads() to after the second one.  The reads then run after other waves may have
passed both barriers, and those waves can already be writing the tile again.  This was seen in a
trial kernel that looped over tiles through one LDS buffer: it gave wrong outputs in a few tiles,
and only from a block's second tile on.  None of the library's kernels rewrites a staged tile
after the reads that a barrier is meant to order, and this test keeps the tell-tale pair out of
the library whatever the compiler does.

The code object is extracted and disassembled as in test_isa_shift64 (no GPU needed).
"""
import re

from test_isa_shift64 import _disassemble

BETWEEN_OK = re.compile(r"^(s_waitcnt|s_nop|s_waitcnt_vscnt|s_waitcnt_lgkmcnt|s_waitcnt_vmcnt)\b")


def adjacent_barriers(disassembly):
    """[(function, line)] for every s_barrier preceded, since the previous s_barrier of the same
    function, only by waits and nops."""
    found, fn, since = [], None, None
    for line in disassembly.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:", line)
        if m:
            fn, since = m.group(1), None
            continue
        ins = line.split("//")[0].strip()
        if not ins:
            continue
        if ins.startswith("s_barrier"):
            if since is not None and all(BETWEEN_OK.match(i) for i in since):
                found.append((fn, ins))
            since = []
        elif since is not None:
            since.append(ins)
    return found


def test_parser_flags_only_empty_barrier_pairs():
    text = ("0000000000001000 <k>:\n"
            "\tds_write_b128 v1, v[2:5]        // 0001\n"
            "\ts_waitcnt lgkmcnt(0)            // 0002\n"
            "\ts_barrier                       // 0003\n"
            "\ts_barrier                       // 0004\n"
            "\tds_read_b128 v[2:5], v1         // 0005\n"
            "\ts_barrier                       // 0006\n"
            "0000000000002000 <j>:\n"
            "\ts_barrier                       // 0007\n")
    assert adjacent_barriers(text) == [("k", "s_barrier")]


def test_no_adjacent_workgroup_barriers(tmp_path):
    dis = _disassemble(tmp_path)
    assert "s_barrier" in dis
    bad = adjacent_barriers(dis)
    assert not bad, "barrier pairs with nothing between them:\n" + "\n".join(f"{f}: {i}" for f, i in bad[:20])
