"""The decode kernel's span walk (span mode of fd_mfma_partial_kernel in
fd_mfma.hip), restated step by step in Python and run on the CPU against the
oracle's cut rule (``oracle.span_ranges``): on random ragged batches every
key is taken once, each piece lands in the slot the rule names, every slot
of every row is written once (by a piece or as padding) and sequences
without keys are padded whole.  Any change to the kernel's walk must be
mirrored here.
"""
import random

import numpy as np
import pytest

import oracle

KB = 16      # keys per block
PIECE = 16   # line positions in front of each (sequence, KV head) pair


def kernel_walk(lens, Lmax, Hkv, nsp, slots, grid):
    """Pieces (b, g, slot, lo, hi, pad_from) and padded empty sequences, as
    the kernel's workgroups 0 .. grid-1 produce them."""
    B = len(lens)

    def clamp(b):
        return max(0, min(Lmax, lens[b]))

    N, nbmax = 0, 0
    for b in range(B):
        nb = (clamp(b) + KB - 1) // KB
        N += Hkv * (PIECE + nb) if nb > 0 else 0
        nbmax = max(nbmax, nb)
    per = (N + nsp - 1) // nsp
    per = max(per, (nbmax + slots - 2) // (slots - 1), 1)
    pieces, padded = [], set()
    for wg in range(grid):
        for b in range(wg, B, grid):
            if clamp(b) == 0:
                padded.add(b)
        st = {"sp": wg, "sb": 0, "sg": 0, "snb": 0, "sL": 0, "sC": 0, "R0": 0, "R1": 0, "more": False}

        def begin_span():
            st["R0"] = st["sp"] * per
            st["R1"] = min(st["R0"] + per, N)
            st["more"] = st["R0"] < st["R1"]
            if not st["more"]:
                return
            st["sC"] = 0
            sb = 0
            while sb < B:
                st["sL"] = clamp(sb)
                st["snb"] = (st["sL"] + KB - 1) // KB
                wseq = Hkv * (PIECE + st["snb"]) if st["snb"] > 0 else 0
                if st["snb"] > 0 and st["sC"] + wseq > st["R0"]:
                    break
                st["sC"] += wseq
                sb += 1
            st["sb"] = sb
            st["sg"] = (st["R0"] - st["sC"]) // (PIECE + st["snb"]) if st["R0"] > st["sC"] else 0

        begin_span()
        while True:
            done = False
            while True:
                if st["more"] and st["sC"] + st["sg"] * (PIECE + st["snb"]) + PIECE < st["R1"]:
                    break
                st["sp"] += grid
                if st["sp"] >= nsp:
                    done = True
                    break
                begin_span()
            if done:
                break
            first = st["sC"] + st["sg"] * (PIECE + st["snb"]) + PIECE
            end = first + st["snb"]
            blo = max(st["R0"], first) - first
            bhi = min(st["R1"], end) - first
            g, b, L = st["sg"], st["sb"], st["sL"]
            s = st["sp"] - first // per
            lo, hi = blo * KB, min(bhi * KB, L)
            pad_from = s + 1 if end <= st["R1"] else slots
            assert 0 <= s < slots and 0 <= lo < hi <= L
            pieces.append((b, g, s, lo, hi, pad_from))
            st["sg"] += 1
            if st["sg"] == Hkv:
                st["sg"] = 0
                st["sC"] += Hkv * (PIECE + st["snb"])
                st["snb"] = 0
                while st["snb"] == 0:
                    st["sb"] += 1
                    if st["sb"] >= B:
                        break
                    st["sL"] = clamp(st["sb"])
                    st["snb"] = (st["sL"] + KB - 1) // KB
                st["more"] = st["sb"] < B
    return pieces, padded


def _cases(n, seed):
    rng = random.Random(seed)
    for _ in range(n):
        B = rng.randint(1, 10)
        Hkv = rng.choice([1, 2, 4, 8])
        slots = rng.randint(2, 9)
        Lmax = rng.choice([0, 16, 100, 3000])
        lens = [rng.choice([0, rng.randint(-3, 40), rng.randint(0, 3200)]) for _ in range(B)]
        nsp = rng.randint(1, 70)
        yield lens, Lmax, Hkv, nsp, slots, rng.randint(1, nsp)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_kernel_walk_follows_the_cut_rule(seed):
    for lens, Lmax, Hkv, nsp, slots, grid in _cases(1000, seed):
        pieces, padded = kernel_walk(lens, Lmax, Hkv, nsp, slots, grid)
        cl = [max(0, min(Lmax, L)) for L in lens]
        lo, hi, _ = oracle.span_ranges(cl, Hkv, nsp, slots, piece_blocks=PIECE)
        got_lo, got_hi = np.zeros_like(lo), np.zeros_like(hi)
        for (b, g, s, a, e, _) in pieces:
            assert got_hi[b, g, s] == 0, "two pieces in one slot"
            got_lo[b, g, s], got_hi[b, g, s] = a, e
        assert np.array_equal(got_lo, lo) and np.array_equal(got_hi, hi), (lens, Lmax, Hkv, nsp, slots, grid)
        assert padded == {b for b, L in enumerate(cl) if L == 0}
        for b, L in enumerate(cl):
            if L == 0:
                continue
            for g in range(Hkv):
                written = []
                for (bb, gg, s, _, _, pad_from) in pieces:
                    if (bb, gg) == (b, g):
                        written += [s] + list(range(pad_from, slots))
                assert sorted(written) == list(range(slots)), "every slot written once"
