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
layouts, lane = 32 hl + col; dequantisation: lane l converts 16-byte code
chunk n * lanes + l).
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


def dequant_chunks(D, odd_first_rule):
    """(row, first bf16 chunk, second bf16 chunk) of each 16-byte code chunk
    q in lane order: code rows of D bytes (CH8 chunks), bf16 rows of 2D."""
    ch8 = D // 16
    out = []
    for q in range(16 * ch8):
        r, c = q // ch8, q % ch8
        odd_first = odd_first_rule(r, c, ch8)
        out.append((r, 2 * c + (1 if odd_first else 0), 2 * c + (0 if odd_first else 1)))
    return out


KERNEL_RULE = lambda r, c, ch8: (c >= ch8 // 2) != (ch8 == 4 and (r & 1) == 1)  # noqa: E731


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sw,name", [(SWF, "decode"), (CSWF, "chunk")])
def test_dequant_writes_conflict_free(D, sw, name):
    ch = 2 * D // 16
    chunks = dequant_chunks(D, KERNEL_RULE)
    for which in (1, 2):
        for n in range(len(chunks) // 64):
            def addr(l, n=n, which=which):
                r, a, b = chunks[n * 64 + l]
                return r * 2 * D + (((a if which == 1 else b) ^ sw(r, ch)) << 4)
            assert not write_b128(addr), (name, D, which, n)


def test_models_see_the_plain_conflicts():
    # The checks can fail: unswizzled transposed reads of 256-byte rows at
    # one chunk pair, and dequantisation writes in plain even/odd order.
    assert tr_read(lambda l: ((l >> 2) & 7) * 256 + 8 * (l & 3))
    plain = dequant_chunks(128, lambda r, c, ch8: False)
    assert write_b128(lambda l: plain[l][0] * 256 + (plain[l][1] << 4))
