"""The oracle's balanced-span split (``oracle.span_ranges``) and its split
form over explicit key ranges (``oracle.attention_ranges``), pinned to what
the definitions fix: a key-by-key recount of the cut rule, the balance the
rule promises, the plain softmax of a slot's keys, and split invariance (any
disjoint ranges covering the visible keys merge to the attention itself).
"""
import math

import numpy as np
import pytest

import oracle
from decode_attention_14_amd.inputs import as_oracle_array, make_inputs

CASES = [
    # lens, Hkv, spans, slots
    ([1000, 77, 0, 640, 33, 2000], 2, 7, 4),
    ([1601, 1732, 2048, 8088, 8049, 512], 8, 64, 7),
    ([16, 17, 15, 1, 0, 0, 32], 4, 5, 3),
    ([0, 0], 2, 3, 2),
    ([4096], 1, 1, 2),
    ([300, 5000, 40, 2222, 900], 3, 1000, 6),
]


PIECE = 16  # line positions in front of each pair: the fixed cost of a piece


def _recount(lens, Hkv, spans, slots, block=16):
    """The cut rule key by key: the line position of block j of pair (b, g)
    is (positions of all earlier pairs with keys, PIECE + their blocks each)
    + PIECE + j; its cut is position // per; its slot is its cut minus the
    cut of the pair's block 0."""
    nb = [-(-L // block) for L in lens]
    total = sum(Hkv * (PIECE + n) for n in nb if n)
    per = max(math.ceil(total / spans), math.ceil(max(nb + [0]) / (slots - 1)), 1)
    slot_of = {}
    pos = 0
    for b, L in enumerate(lens):
        for g in range(Hkv):
            if not nb[b]:
                continue
            first = pos + PIECE
            for j in range(L):
                slot_of[(b, g, j)] = (first + j // block) // per - first // per
            pos = first + nb[b]
    return slot_of, per, total


@pytest.mark.parametrize("lens,Hkv,spans,slots", CASES)
def test_span_ranges_match_a_key_by_key_recount(lens, Hkv, spans, slots):
    lo, hi, per = oracle.span_ranges(lens, Hkv, spans, slots, piece_blocks=PIECE)
    slot_of, per2, total = _recount(lens, Hkv, spans, slots)
    assert per == per2
    for b, L in enumerate(lens):
        for g in range(Hkv):
            got = {}
            for i in range(slots):
                for j in range(lo[b, g, i], hi[b, g, i]):
                    assert (b, g, j) not in got
                    got[(b, g, j)] = i
            assert got == {key: s for key, s in slot_of.items() if key[:2] == (b, g)}
            used = [i for i in range(slots) if hi[b, g, i] > lo[b, g, i]]
            assert used == list(range(len(used))), "a pair's pieces fill slots 0, 1, ..."
            assert all(lo[b, g, i] % 16 == 0 for i in used)


@pytest.mark.parametrize("lens,Hkv,spans,slots", CASES)
def test_span_cuts_are_balanced(lens, Hkv, spans, slots):
    _, per, total = _recount(lens, Hkv, spans, slots)
    nb = [-(-L // 16) for L in lens]
    if per == max(math.ceil(total / spans), 1):
        # every cut but the last holds exactly per blocks: the line is cut
        # into ceil(total / per) <= spans pieces
        assert math.ceil(total / per) <= spans
    # no pair ever needs more slots than there are
    assert all(math.ceil(n / per) + 1 <= slots or n == 0 for n in nb)


def _inputs(lens, Hkv, q_len=1, D=64, seed=1234):
    Lmax = max(max(lens), q_len, 1)
    q, k, v, cl = make_inputs(len(lens), 2 * Hkv, Hkv, D, q_len, Lmax, "bf16", seed, cache_lens=lens)
    return as_oracle_array(q), as_oracle_array(k), as_oracle_array(v), cl.numpy()


@pytest.mark.parametrize("q_len", [1, 3])
def test_span_partials_merge_to_the_attention(q_len):
    lens = [300, 77, 0, 640, 33, 100]
    q, k, v, cl = _inputs(lens, 2, q_len)
    cl = np.maximum(cl, np.where(cl > 0, q_len, 0)).astype(np.int32)
    lo, hi, _ = oracle.span_ranges(cl, 2, 9, 5, piece_blocks=PIECE)
    out, lse, _, _, _ = oracle.attention_ranges(q, k, v, cl, 0.125, lo, hi)
    ref_out, ref_lse = oracle.attention(q, k, v, cl, 0.125)
    assert np.array_equal(np.isinf(lse), np.isinf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(lse[fin] - ref_lse[fin])) < 1e-12
    assert np.max(np.abs(out - ref_out)) < 1e-12
    # a range that drops one key changes the result (the merge is not blind)
    lo2 = lo.copy()
    b, g, i = 0, 0, 0
    lo2[b, g, i] += 1
    out2, _, _, _, _ = oracle.attention_ranges(q, k, v, cl, 0.125, lo2, hi)
    assert np.max(np.abs(out2 - ref_out)) > 1e-6


def test_range_partials_are_the_plain_softmax_of_their_keys():
    lens = [200, 45]
    q, k, v, cl = _inputs(lens, 1, 1, 64, seed=99)
    lo = np.array([[[0, 64, 0]], [[16, 0, 0]]], np.int32)
    hi = np.array([[[64, 200, 0]], [[45, 16, 0]]], np.int32)
    _, _, o_p, m_p, l_p = oracle.attention_ranges(q, k, v, cl, 0.125, lo, hi)
    bf = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    Q, K, V = bf(q), bf(k), bf(v)
    for b in range(2):
        for h in range(2):
            for i in range(3):
                a, e = lo[b, 0, i], hi[b, 0, i]
                if a >= e:
                    assert m_p[b, h, 0, i] == -np.inf and l_p[b, h, 0, i] == -np.inf
                    continue
                s = 0.125 * (K[b, 0, a:e] @ Q[b, h, 0])
                m = s.max()
                p = np.exp(s - m)
                assert abs(m_p[b, h, 0, i] - m) < 1e-12
                assert abs(l_p[b, h, 0, i] - (m + math.log(p.sum()))) < 1e-12
                assert np.max(np.abs(o_p[b, h, 0, i] - (p / p.sum()) @ V[b, 0, a:e])) < 1e-12


def test_range_form_equals_the_tile_form_on_tile_ranges():
    lens = [1000, 77, 0, 640]
    q, k, v, cl = _inputs(lens, 2, 1, 64, seed=5)
    T, S = 256, 4
    lo = np.zeros((4, 2, S), np.int32)
    hi = np.zeros_like(lo)
    for b, L in enumerate(lens):
        for i in range(-(-L // T)):
            lo[b, :, i], hi[b, :, i] = i * T, min(L, (i + 1) * T)
    r = oracle.attention_ranges(q, k, v, cl, 0.125, lo, hi)
    t = oracle.attention_split(q, k, v, cl, 0.125, tile_len=T, slots=S)
    for x, y in zip(r, t):
        assert np.array_equal(np.isinf(x), np.isinf(y))
        fin = np.isfinite(y)
        assert np.max(np.abs(x[fin] - y[fin])) < 1e-12
