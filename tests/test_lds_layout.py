"""LDS layout of the matrix-core kernels: the XOR swizzles of 16-byte chunks
(``swf`` in fd_mfma.hip, ``cswf`` in fd_chunk.hip), read from the kernel
sources themselves, checked on the CPU against the operand read patterns the
kernels issue.

Bank model the layouts are designed against: 64 banks of 4 bytes; a
``ds_read_b128`` is served 16 lanes per pass and a ``ds_read_b64`` /
``ds_read_b64_tr_b16`` 32 lanes per pass, so a pass that moves 256 bytes is
conflict-free exactly when its lanes touch 64 distinct banks.  The lane ->
(row, chunk) maps below restate the address arithmetic of the kernels'
operand loads (decode: 16x16 layouts, lane = 16 grp + col; chunk: 32x32
layouts, lane = 32 hl + col).
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "decode_attention_14_amd", "csrc")
BANKS, BANK_BYTES = 64, 4


def load_swizzle(fname, name):
    """The body of `template <int CH> int name(int r)` as a Python function
    of (r, CH); its statements are C integer expressions with the same
    meaning in Python for non-negative operands."""
    src = open(os.path.join(CSRC, fname)).read()
    m = re.search(r"int " + name + r"\(int r\) \{\n(.*?)\n\}", src, re.S)
    assert m, f"{name} not found in {fname}"
    lines = ["def f(r, CH):"]
    for st in m.group(1).strip().split("\n"):
        st = st.strip().rstrip(";")
        st = re.sub(r"^if constexpr \((.*?)\) return (.*)$", r"if \1: return \2", st)
        st = re.sub(r"^const int (\w+) = ", r"\1 = ", st)
        lines.append("    " + st)
    ns = {}
    exec("\n".join(lines), ns)
    return ns["f"]


SWF = load_swizzle("fd_mfma.hip", "swf")
CSWF = load_swizzle("fd_chunk.hip", "cswf")


def conflict_free(addrs, nbytes):
    banks = []
    for a in addrs:
        assert a % nbytes == 0
        banks += [(a // BANK_BYTES + k) % BANKS for k in range(nbytes // BANK_BYTES)]
    return len(banks) == len(set(banks))


def passes(addr_of_lane, lanes_per_pass, nbytes):
    bad = []
    for p in range(64 // lanes_per_pass):
        lanes = range(p * lanes_per_pass, (p + 1) * lanes_per_pass)
        if not conflict_free([addr_of_lane(l) for l in lanes], nbytes):
            bad.append(p)
    return bad


@pytest.mark.parametrize("sw", [SWF, CSWF], ids=["swf", "cswf"])
@pytest.mark.parametrize("CH", [8, 16])
def test_swizzle_permutes_each_row(sw, CH):
    # Every row's chunks land on distinct slots (XOR by a value below CH),
    # and the map depends on the row only modulo 16.
    for r in range(64):
        x = sw(r, CH)
        assert 0 <= x < CH
        assert sorted(c ^ x for c in range(CH)) == list(range(CH))
        assert x == sw(r % 16, CH)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_operand_reads_conflict_free(D):
    rowb, ch = 2 * D, 2 * D // 16

    def swz(r, c):
        return r * rowb + ((c ^ SWF(r, ch)) << 4)

    for ks in range(D // 32):  # K: A operand of the 16x16x32 score product
        assert not passes(lambda l: swz(l & 15, (l >> 4) + 4 * ks), 16, 16), (D, ks)
    for db in range(D // 16):  # V^T: 16-lane transposed reads, 4 rows x 2 chunks

        def v_addr(l, db=db):
            grp, col = l >> 4, l & 15
            r, q4 = 4 * grp + (col >> 2), col & 3
            return swz(r, 2 * db + (q4 >> 1)) + 8 * (q4 & 1)

        assert not passes(v_addr, 32, 8), (D, db)


@pytest.mark.parametrize("D", [64, 128])
def test_chunk_operand_reads_conflict_free(D):
    rowb, ch = 2 * D, 2 * D // 16

    def cswz(r, c):
        return r * rowb + ((c ^ CSWF(r, ch)) << 4)

    for ks in range(D // 16):  # K: A operand of the 32x32x16 score product
        assert not passes(lambda l: cswz(l & 31, 2 * ks + (l >> 5)), 16, 16), (D, ks)
    for db in range(D // 32):
        for t in range(2):
            for step in range(2):  # the second 16-key step reads 16 rows further

                def v_addr(l, db=db, t=t, step=step):
                    hl, g16, i16 = l >> 5, l >> 4, l & 15
                    q4 = i16 & 3
                    r = 8 * t + 4 * hl + (i16 >> 2)
                    return (cswz(r, (32 * db + 16 * (g16 & 1)) // 8 + (q4 >> 1)) + 8 * (q4 & 1)
                            + step * 16 * rowb)

                assert not passes(v_addr, 32, 8), (D, db, t, step)


def test_unswizzled_layout_conflicts():
    # The check itself: without the swizzle, the K reads (16 rows at one
    # chunk, 256-byte rows) all fall into the same four banks.
    assert passes(lambda l: (l & 15) * 256 + 16 * (l >> 4), 16, 16)
