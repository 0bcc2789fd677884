"""LDS layout of the matrix-core kernels: the XOR swizzles of 16-byte chunks
(``swf`` in fd_mfma.hip, ``cswf`` in fd_chunk.hip), read from the kernel
sources themselves, checked on the CPU against the kernels' LDS access
patterns.

Bank behaviour on gfx950, fitted to SQ_LDS_BANK_CONFLICT counts of single-wave
probes over strided and permuted lane -> address patterns (each model below
reproduces every measured count of its instruction):
  * ``ds_read_b64`` / ``ds_read_b64_tr_b16``: 32 consecutive lanes per LDS
    cycle over 64 banks of 4 bytes (256 bytes);
  * ``ds_write_b128``: 8 consecutive lanes per cycle over 128 bytes of banks.
A pass is conflict-free when no two of its lanes touch the same bank at
different addresses.  ``ds_read_b128`` follows no such simple pass model; the
K-operand maps were chosen by measuring the kernels themselves.
The lane -> (row, chunk) maps below restate the address arithmetic of the
kernels (decode: 16x16 layouts, lane = 16 grp + col; chunk kernel: 32x32
layouts, lane = 32 hl + col; dequantisation: lane l converts 8-byte code
unit n * lanes + l into one 16-byte bf16 chunk).
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "decode_attention_14_amd", "csrc")
BANK_BYTES = 4


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


def load_merge_at():
    """merge_at(r, d) of fd_chunk.hip (float offset of dims d .. d + 3 of row
    r in a row group's merge block) as a Python function of (r, d, D)."""
    src = open(os.path.join(CSRC, "fd_chunk.hip")).read()
    m = re.search(r"int merge_at\(int r, int d\) \{\n\s*return (.*?);\n\}", src, re.S)
    assert m, "merge_at not found in fd_chunk.hip"
    return eval("lambda r, d, D: " + m.group(1))


MERGE_AT = load_merge_at()


def conflict_free(addrs, nbytes, window):
    banks = {}
    for a in addrs:
        assert a % nbytes == 0
        for k in range(nbytes // BANK_BYTES):
            word = a // BANK_BYTES + k
            bank = word % (window // BANK_BYTES)
            if banks.setdefault(bank, word) != word:
                return False
    return True


def passes(addr_of_lane, lanes_per_pass, nbytes, window):
    """Indices of the passes that have a bank conflict."""
    return [p for p in range(64 // lanes_per_pass)
            if not conflict_free([addr_of_lane(l) for l in range(p * lanes_per_pass, (p + 1) * lanes_per_pass)],
                                 nbytes, window)]


def tr_read(f):  # ds_read_b64_tr_b16
    return passes(f, 32, 8, 256)


def write_b128(f):
    return passes(f, 8, 16, 128)


@pytest.mark.parametrize("sw", [SWF, CSWF], ids=["swf", "cswf"])
@pytest.mark.parametrize("CH", [8, 16])
def test_swizzle_permutes_each_row(sw, CH):
    # Every row's chunks land on distinct slots (XOR by a value below CH), the
    # map depends on the row only modulo 16, and it is a bijection on the
    # rows that share a bank cycle (16 rows of 256 bytes, or row pairs).
    for r in range(64):
        x = sw(r, CH)
        assert 0 <= x < CH
        assert sorted(c ^ x for c in range(CH)) == list(range(CH))
        assert x == sw(r % 16, CH)
    rows = range(16) if CH == 16 else range(0, 16, 2)
    assert len({sw(r, CH) for r in rows}) == len(rows)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_v_reads_conflict_free(D):
    rowb, ch = 2 * D, 2 * D // 16

    def swz(r, c):
        return r * rowb + ((c ^ SWF(r, ch)) << 4)

    for db in range(D // 16):  # V^T: 4 rows x an even/odd chunk pair per 16 lanes

        def v_addr(l, db=db):
            grp, col = l >> 4, l & 15
            r, q4 = 4 * grp + (col >> 2), col & 3
            return swz(r, 2 * db + (q4 >> 1)) + 8 * (q4 & 1)

        assert not tr_read(v_addr), (D, db)


@pytest.mark.parametrize("D", [64, 128])
def test_chunk_v_reads_conflict_free(D):
    rowb, ch = 2 * D, 2 * D // 16

    def cswz(r, c):
        return r * rowb + ((c ^ CSWF(r, ch)) << 4)

    for db in range(D // 32):
        for t in range(2):
            for step in range(2):  # the second 16-key step reads 16 rows further

                def v_addr(l, db=db, t=t, step=step):
                    hl, g16, i16 = l >> 5, l >> 4, l & 15
                    q4 = i16 & 3
                    r = 8 * t + 4 * hl + (i16 >> 2)
                    return (cswz(r, (32 * db + 16 * (g16 & 1)) // 8 + (q4 >> 1)) + 8 * (q4 & 1)
                            + step * 16 * rowb)

                assert not tr_read(v_addr), (D, db, t, step)


@pytest.mark.parametrize("D", [64, 128])
def test_chunk_merge_block_layout(D):
    # Each row's 16-byte chunks are permuted within the row (the block holds
    # 32 rows x D floats exactly), and the key-half merge's float4 writes --
    # lane (hl, col) writes dims 32 db + 8 a4 + 4 hl of row col -- are
    # conflict-free.
    for r in range(32):
        offs = sorted(MERGE_AT(r, d, D) for d in range(0, D, 4))
        assert offs == list(range(r * D, (r + 1) * D, 4)), (D, r)
    for db in range(D // 32):
        for a4 in range(4):
            def addr(l, db=db, a4=a4):
                hl, col = l >> 5, l & 31
                return 4 * MERGE_AT(col, 32 * db + 8 * a4 + 4 * hl, D)
            assert not write_b128(addr), (D, db, a4)


def dequant_units(D, code_swz):
    """(row, bf16 chunk) written for each 8-byte code unit u in lane order:
    code rows of D bytes whose 16-byte chunks are XOR-swizzled by
    code_swz(row) (the decode kernel's ring; 0 for the chunk kernel's plain
    code stage), bf16 rows of 2D bytes (16-byte chunk c = dims 8c .. 8c + 7)."""
    upr = D // 8
    out = []
    for u in range(16 * upr):
        r, pu = u // upr, u % upr
        out.append((r, (((pu >> 1) ^ code_swz(r)) << 1) | (pu & 1)))
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sw,name", [(SWF, "decode"), (CSWF, "chunk")])
def test_dequant_writes_conflict_free(D, sw, name):
    # Any code swizzle that XORs a row's chunk index with a value below its
    # chunk count keeps each write cycle conflict-free: the decode kernel's
    # cswz8 is one of these, the chunk kernel's plain code stage is k = 0.
    ch, ch8 = 2 * D // 16, D // 16
    for k in range(ch8):
        units = dequant_units(D, lambda r, k=k: (5 * r + k) % ch8)
        for n in range(len(units) // 64):
            def addr(l, n=n):
                r, c = units[n * 64 + l]
                return r * 2 * D + ((c ^ sw(r, ch)) << 4)
            assert not write_b128(addr), (name, D, k, n)


def test_models_see_the_plain_conflicts():
    # The checks can fail: unswizzled transposed reads of 256-byte rows at
    # one chunk pair, and dequantisation writes of 16-byte code chunks in even/odd
    # order.
    assert tr_read(lambda l: ((l >> 2) & 7) * 256 + 8 * (l & 3))
    # (Lane l converting 16-byte code chunk l and writing its even bf16 chunk
    # first: the 8 lanes of a cycle hit only 4 chunks modulo 8.)
    assert write_b128(lambda l: (l // 8) * 256 + ((2 * (l % 8)) << 4))
