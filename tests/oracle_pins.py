"""Checks that pin the fp64 oracle to facts outside itself.

Each ``check_*`` takes a loaded oracle library (the real one, or a copy with a
planted mistake) and raises ``AssertionError`` when the oracle disagrees with:
  * hand-derived closed-form results (``tests/golden/closed_forms.json``);
  * torch's own attention routine (``scaled_dot_product_attention`` and
    ``logsumexp`` in float64 on the CPU), an implementation that shares
    nothing with the oracle;
  * invariants of the method: split-count invariance of the merged result,
    the one-split case, the sequential rescaling form, partial statistics,
    merging partials of disjoint key sets, identical keys, zero scale, one
    dominant key, convexity, linearity in V, GQA as MHA with repeated K/V,
    a chunk row as a decode step, poison beyond the cache length, exact
    bf16 widening.
The pins are chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one mask) fails at least
one of them; ``test_oracle_mutants.py`` plants such slips to prove it.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from decode_attention_14_amd.inputs import as_oracle_array, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def _arr(x):
    return np.array(x, dtype=np.float64)


def _lse_arr(x):
    return np.array([[[-math.inf if e == "-inf" else e for e in row] for row in blk] for blk in x],
                    dtype=np.float64)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b) and np.array_equal(a[inf_a], b[inf_b]), f"{what}: infinities differ"
    fin = ~inf_a
    assert not np.isnan(a).any(), f"{what}: NaN in oracle result"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rel_close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    if fin.any():
        scale = max(1.0, float(np.max(np.abs(b[fin]))))
        err = float(np.max(np.abs(a[fin] - b[fin])))
        assert err <= rtol * scale, f"{what}: error {err:.3e} > {rtol:.1e} x {scale:.2f}"


# --------------------------------------------------------------------------
# Golden closed forms


def check_golden(lib):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.array(c["q"], np.float32)
        k = np.array(c["k"], np.float32)
        v = np.array(c["v"], np.float32)
        lens = np.array(c["cache_lens"], np.int32)
        exp_out, exp_lse, tol = _arr(c["out"]), _lse_arr(c["lse"]), c["tol"]
        out, lse = oracle.attention(q, k, v, lens, c["scale"], lib=lib)
        _close(out, exp_out, tol, c["name"] + " out")
        _close(lse, exp_lse, tol, c["name"] + " lse")
        for ns in (1, 2):
            so, sl, *_ = oracle.attention_split(q, k, v, lens, c["scale"], num_splits=ns, lib=lib)
            _close(so, exp_out, tol, f"{c['name']} split{ns} out")
            _close(sl, exp_lse, tol, f"{c['name']} split{ns} lse")
        for blk in (1, 2):
            qo, ql = oracle.attention_sequential(q, k, v, lens, c["scale"], block=blk, lib=lib)
            _close(qo, exp_out, tol, f"{c['name']} seq{blk} out")
            _close(ql, exp_lse, tol, f"{c['name']} seq{blk} lse")


# --------------------------------------------------------------------------
# Library attention routine (torch, float64, CPU)


def library_attention(q, k, v, lens, scale):
    """Reference via torch's SDPA with an explicit bottom-right causal mask."""
    q = torch.as_tensor(q, dtype=torch.float64)
    k = torch.as_tensor(k, dtype=torch.float64)
    v = torch.as_tensor(v, dtype=torch.float64)
    B, Hq, T, D = q.shape
    n_rep = Hq // k.shape[1]
    kk = k.repeat_interleave(n_rep, dim=1)
    vv = v.repeat_interleave(n_rep, dim=1)
    out = torch.zeros(B, Hq, T, D, dtype=torch.float64)
    lse = torch.full((B, Hq, T), -math.inf, dtype=torch.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        pos = torch.arange(L)
        limit = torch.arange(T) + (L - T)            # last visible key per row
        mask = pos[None, :] <= limit[:, None]        # [T, L]
        rows = mask.any(dim=1)
        if not rows.any():
            continue
        qb = q[b:b + 1, :, rows]
        mb = mask[rows]
        kb = kk[b:b + 1, :, :L].contiguous()
        vb = vv[b:b + 1, :, :L].contiguous()
        o = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=mb, scale=float(scale))
        sc = torch.matmul(qb, kb.transpose(-1, -2).contiguous()) * float(scale)
        sc = sc.masked_fill(~mb, -math.inf)
        out[b][:, rows] = o[0]
        lse[b][:, rows] = torch.logsumexp(sc, dim=-1)[0]
    return out.numpy(), lse.numpy()


def _widen(t):
    return t.to(torch.float64).numpy()


def _library_cases():
    # (B, Hq, Hkv, D, q_len, Lmax, dtype, seed, lens)
    return [
        (1, 2, 2, 8, 1, 5, "f32", 1, [5]),
        (2, 4, 2, 16, 1, 11, "f32", 2, [5, 11]),
        (2, 8, 2, 16, 3, 9, "bf16", 3, [9, 4]),
        (3, 4, 1, 8, 4, 12, "bf16", 4, [12, 7, 4]),
        (1, 6, 3, 32, 5, 20, "f32", 5, [3]),
    ]


def check_library(lib):
    for (B, Hq, Hkv, D, T, Lmax, dt, seed, lens) in _library_cases():
        q, k, v, cl = make_inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, cache_lens=lens)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        out, lse = oracle.attention(as_oracle_array(q), as_oracle_array(k), as_oracle_array(v),
                                    cl.numpy(), scale, lib=lib)
        ref_out, ref_lse = library_attention(_widen(q), _widen(k), _widen(v), lens, scale)
        _close(out, ref_out, 1e-12, f"library case {seed} out")
        _close(lse, ref_lse, 1e-12, f"library case {seed} lse")


# --------------------------------------------------------------------------
# Invariants of the split / merge method


def _rand_case(seed, B=2, Hq=4, Hkv=2, D=16, T=1, Lmax=37, lens=(37, 23), dt="f32"):
    q, k, v, cl = make_inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, cache_lens=list(lens))
    return (as_oracle_array(q), as_oracle_array(k), as_oracle_array(v), cl.numpy(),
            float(np.float32(1.0 / math.sqrt(D))))


def check_split_invariance(lib):
    for T in (1, 3):
        q, k, v, lens, scale = _rand_case(11 + T, T=T)
        out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
        for ns in (1, 2, 3, 4, 7, 37):
            so, sl, *_ = oracle.attention_split(q, k, v, lens, scale, num_splits=ns, lib=lib)
            _rel_close(so, out, 1e-12, f"split{ns} out (q_len={T})")
            _rel_close(sl, lse, 1e-12, f"split{ns} lse (q_len={T})")
        for tile in (1, 5, 16, 64):
            so, sl, *_ = oracle.attention_split(q, k, v, lens, scale, tile_len=tile, lib=lib)
            _rel_close(so, out, 1e-12, f"tile{tile} out (q_len={T})")
            _rel_close(sl, lse, 1e-12, f"tile{tile} lse (q_len={T})")


def check_one_split_partials(lib):
    q, k, v, lens, scale = _rand_case(21, T=2)
    out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
    so, sl, op, mp, lp = oracle.attention_split(q, k, v, lens, scale, num_splits=1, lib=lib)
    _rel_close(op[..., 0, :], out, 1e-12, "one-split partial o")
    _rel_close(lp[..., 0], lse, 1e-12, "one-split partial lse")


def check_sequential(lib):
    for T in (1, 4):
        q, k, v, lens, scale = _rand_case(31 + T, T=T)
        out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
        for blk in (1, 3, 8, 256):
            so, sl = oracle.attention_sequential(q, k, v, lens, scale, block=blk, lib=lib)
            _rel_close(so, out, 1e-12, f"sequential block {blk} out")
            _rel_close(sl, lse, 1e-12, f"sequential block {blk} lse")


def check_partial_stats(lib):
    q, k, v, lens, scale = _rand_case(41, T=3)
    _, _, op, mp, lp = oracle.attention_split(q, k, v, lens, scale, tile_len=8, lib=lib)
    B, Hq, T = q.shape[0], q.shape[1], q.shape[2]
    S = mp.shape[-1]
    for b in range(B):
        L = int(lens[b])
        for t in range(T):
            nvis = max(0, min(L, L - T + t + 1))
            for s in range(S):
                n_s = max(0, min(nvis, (s + 1) * 8) - s * 8)
                m, ls = mp[b, :, t, s], lp[b, :, t, s]
                if n_s == 0:
                    assert np.all(m == -np.inf) and np.all(ls == -np.inf), "empty tile must be -inf"
                    assert np.all(op[b, :, t, s] == 0), "empty tile output must be 0"
                else:
                    assert np.all(m <= ls + 1e-12), "tile lse below tile max"
                    assert np.all(ls <= m + math.log(n_s) + 1e-12), "tile lse above max + ln n"


def check_merge_disjoint(lib):
    """Merging partials of two disjoint key sets equals attention over their union."""
    q, k, v, lens, scale = _rand_case(51, B=1, lens=(37,), T=1)
    out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
    cut = 13
    k1, v1 = np.ascontiguousarray(k[:, :, :cut]), np.ascontiguousarray(v[:, :, :cut])
    k2, v2 = np.ascontiguousarray(k[:, :, cut:]), np.ascontiguousarray(v[:, :, cut:])
    o1, l1 = oracle.attention(q, k1, v1, [cut], scale, lib=lib)
    o2, l2 = oracle.attention(q, k2, v2, [37 - cut], scale, lib=lib)
    o_part = np.stack([o1, o2, np.full_like(o1, np.nan)], axis=-2)   # third slot empty
    l_part = np.stack([l1, l2, np.full_like(l1, -np.inf)], axis=-1)
    mo, ml = oracle.merge_lse(o_part, l_part, lib=lib)
    _rel_close(mo, out, 1e-12, "merge of disjoint halves out")
    _rel_close(ml, lse, 1e-12, "merge of disjoint halves lse")
    # Closed forms of the merge itself: equal lse -> plain mean, LSE = a + ln 2;
    # all slots empty -> 0 and -inf.
    a = 0.75
    po = np.array([[[1.0, -2.0], [3.0, 6.0]]])
    pl = np.array([[a, a]])
    mo, ml = oracle.merge_lse(po, pl, lib=lib)
    _close(mo, np.array([[2.0, 2.0]]), 1e-15, "merge equal weights out")
    _close(ml, np.array([a + math.log(2.0)]), 1e-15, "merge equal weights lse")
    mo, ml = oracle.merge_lse(po, np.array([[-np.inf, -np.inf]]), lib=lib)
    _close(mo, np.zeros((1, 2)), 0.0, "merge empty out")
    assert ml[0] == -np.inf, "merge of empty slots must give -inf"
    # lse 0 and ln 3 -> weights 1/4, 3/4.
    mo, ml = oracle.merge_lse(po, np.array([[0.0, math.log(3.0)]]), lib=lib)
    _close(mo, np.array([[2.5, 4.0]]), 1e-15, "merge 1:3 out")
    _close(ml, np.array([math.log(4.0)]), 1e-15, "merge 1:3 lse")


def check_closed_forms(lib):
    rng = np.random.Generator(np.random.PCG64(61))
    B, Hq, Hkv, D, Lmax = 1, 2, 1, 8, 10
    q = rng.standard_normal((B, Hq, 1, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Lmax, D), dtype=np.float32)
    lens = np.array([7], np.int32)
    # identical keys: out = mean of the visible V rows, lse = s + ln n
    krow = rng.standard_normal(D, dtype=np.float32)
    k = np.broadcast_to(krow, (B, Hkv, Lmax, D)).copy()
    scale = 0.5
    out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
    mean_v = v[0, 0, :7].astype(np.float64).mean(axis=0)
    for h in range(Hq):
        s = scale * float(np.dot(q[0, h, 0].astype(np.float64), krow.astype(np.float64)))
        _close(out[0, h, 0], mean_v, 1e-12, "identical keys out")
        _close(lse[0, h, 0], s + math.log(7), 1e-12, "identical keys lse")
    # zero scale: the same for any keys, lse = ln n
    k2 = rng.standard_normal((B, Hkv, Lmax, D), dtype=np.float32)
    out, lse = oracle.attention(q, k2, v, lens, 0.0, lib=lib)
    _close(out[0, :, 0], np.broadcast_to(mean_v, (Hq, D)), 1e-12, "zero scale out")
    _close(lse[0, :, 0], np.full(Hq, math.log(7)), 1e-12, "zero scale lse")
    # one dominant key: q . k_j = 40 * |q|^2 beats every other score by > 30
    j = 4
    k3 = k2.copy() * 0.01
    k3[0, 0, j] = 40.0 * q[0, 0, 0]
    out, lse = oracle.attention(q[:, :1], k3, v, lens, 1.0, lib=lib)
    _close(out[0, 0, 0], v[0, 0, j], 1e-9, "dominant key out")
    # convexity and linearity in V on random data
    q4, k4, v4, lens4, sc4 = _rand_case(62, T=2)
    out, _ = oracle.attention(q4, k4, v4, lens4, sc4, lib=lib)
    for b in range(out.shape[0]):
        L = int(lens4[b])
        lo = v4[b, :, :L].min(axis=1)
        hi = v4[b, :, :L].max(axis=1)
        n_rep = out.shape[1] // lo.shape[0]
        lo = np.repeat(lo, n_rep, axis=0)[:, None, :]
        hi = np.repeat(hi, n_rep, axis=0)[:, None, :]
        assert np.all(out[b] >= lo - 1e-12) and np.all(out[b] <= hi + 1e-12), "output outside hull of V"
    ints = np.random.Generator(np.random.PCG64(63))
    va = ints.integers(-8, 9, size=v4.shape).astype(np.float32)
    vb = ints.integers(-8, 9, size=v4.shape).astype(np.float32)
    oa, _ = oracle.attention(q4, k4, va, lens4, sc4, lib=lib)
    ob, _ = oracle.attention(q4, k4, vb, lens4, sc4, lib=lib)
    oab, _ = oracle.attention(q4, k4, (2 * va + vb).astype(np.float32), lens4, sc4, lib=lib)
    _rel_close(oab, 2 * oa + ob, 1e-12, "linearity in V")


def check_gqa_equiv(lib):
    q, k, v, lens, scale = _rand_case(71, Hq=8, Hkv=2, T=2)
    out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
    kr = np.ascontiguousarray(np.repeat(k, 4, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, 4, axis=1))
    mo, ml = oracle.attention(q, kr, vr, lens, scale, lib=lib)
    _close(out, mo, 0.0, "GQA vs repeated-KV MHA out")
    _close(lse, ml, 0.0, "GQA vs repeated-KV MHA lse")


def check_chunk_rows_as_decode(lib):
    T = 5
    q, k, v, lens, scale = _rand_case(81, T=T, lens=(37, 9))
    out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
    for b in range(q.shape[0]):
        L = int(lens[b])
        for t in range(T):
            qt = np.ascontiguousarray(q[b:b + 1, :, t:t + 1])
            kb = np.ascontiguousarray(k[b:b + 1])
            vb = np.ascontiguousarray(v[b:b + 1])
            do, dl = oracle.attention(qt, kb, vb, [L - T + t + 1], scale, lib=lib)
            _close(out[b, :, t], do[0, :, 0], 0.0, f"chunk row {t} vs decode out")
            _close(lse[b, :, t], dl[0, :, 0], 0.0, f"chunk row {t} vs decode lse")


def check_poison(lib):
    for dt in ("f32", "bf16"):
        q, k, v, lens, scale = _rand_case(91, dt=dt, lens=(20, 3), T=2)
        out, lse = oracle.attention(q, k, v, lens, scale, lib=lib)
        kp, vp = k.copy(), v.copy()
        bad = np.float32(np.nan) if dt == "f32" else np.uint16(0x7FC0)
        inf = np.float32(np.inf) if dt == "f32" else np.uint16(0x7F80)
        for b, L in enumerate(lens.tolist()):
            kp[b, :, L:] = bad
            vp[b, :, L:] = inf
        po, pl = oracle.attention(q, kp, vp, lens, scale, lib=lib)
        _close(po, out, 0.0, f"poison beyond length out ({dt})")
        _close(pl, lse, 0.0, f"poison beyond length lse ({dt})")
        for ns in (1, 3):
            so, sl, *_ = oracle.attention_split(q, kp, vp, lens, scale, num_splits=ns, lib=lib)
            _rel_close(so, out, 1e-12, f"poison split{ns} out ({dt})")


def check_bf16_widening(lib):
    """bf16 bit patterns widen exactly: same result as the float32 of those values."""
    q, k, v, cl = make_inputs(2, 4, 2, 16, 2, 13, "bf16", 101, cache_lens=[13, 6])
    scale = 0.25
    ob, lb = oracle.attention(as_oracle_array(q), as_oracle_array(k), as_oracle_array(v),
                              cl.numpy(), scale, lib=lib)
    of, lf = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                              cl.numpy(), scale, lib=lib)
    _close(ob, of, 0.0, "bf16 vs widened f32 out")
    _close(lb, lf, 0.0, "bf16 vs widened f32 lse")
    # a known pattern: 0x3FC0 is 1.5, 0xC040 is -3.0
    one = np.zeros((1, 1, 1, 2), np.uint16)
    one[..., 0] = 0x3FC0
    kk = np.zeros((1, 1, 1, 2), np.uint16)
    vv = np.zeros((1, 1, 1, 2), np.uint16)
    vv[..., 1] = 0xC040
    kk[..., 0] = 0x3FC0
    o, l = oracle.attention(one, kk, vv, [1], 1.0, lib=lib)
    _close(o, np.array([[[[0.0, -3.0]]]]), 0.0, "bf16 pattern out")
    _close(l, np.array([[[2.25]]]), 0.0, "bf16 pattern lse")


ALL_CHECKS = [
    check_golden,
    check_library,
    check_split_invariance,
    check_one_split_partials,
    check_sequential,
    check_partial_stats,
    check_merge_disjoint,
    check_closed_forms,
    check_gqa_equiv,
    check_chunk_rows_as_decode,
    check_poison,
    check_bf16_widening,
]
