"""fp64 CPU oracle for split-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library and its Python binding never import it.

The arithmetic lives in ``fd_oracle.c`` (plain C, double precision, one
thread per independent (batch, head, query-position) row).  This module only
builds that file with gcc, loads it with ctypes and marshals numpy arrays.

Inputs are numpy arrays holding the exact values the GPU reads:
  * fp32 tensors as ``np.float32``;
  * bf16 tensors as their raw bit patterns, ``np.uint16``.
Outputs are ``np.float64``.

Layouts: q/out ``[B, Hq, q_len, D]``, k/v ``[B, Hkv, Lmax, D]``,
cache_lens ``[B]`` int32, lse ``[B, Hq, q_len]``, partials
``[B, Hq, q_len, S, D]`` and ``[B, Hq, q_len, S]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(out_path: str = _LIB, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread",
           *extra_flags, "-o", out_path, src_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _declare(lib):
    i32, dbl, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.orc_attention.argtypes = [i32] * 7 + [vp, vp, vp, vp, dbl, vp, vp, i32]
    lib.orc_attention.restype = i32
    lib.orc_attention_split.argtypes = ([i32] * 7 + [vp, vp, vp, vp, dbl, i32, i32, i32]
                                        + [vp] * 5 + [i32])
    lib.orc_attention_split.restype = i32
    lib.orc_attention_sequential.argtypes = [i32] * 7 + [vp, vp, vp, vp, dbl, i32, vp, vp, i32]
    lib.orc_attention_sequential.restype = i32
    lib.orc_attention_ranges.argtypes = ([i32] * 7 + [vp, vp, vp, vp, dbl, i32, vp, vp]
                                         + [vp] * 5 + [i32])
    lib.orc_attention_ranges.restype = i32
    lib.orc_merge_lse.argtypes = [ctypes.c_long, i32, i32, vp, vp, vp, vp]
    lib.orc_merge_lse.restype = i32
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _prep(q, k, v, cache_lens):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dtype == np.float32:
        code = 0
    elif q.dtype == np.uint16:
        code = 1
    else:
        raise TypeError("inputs must be float32 values or uint16 bf16 bit patterns")
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,q_len,D]; k and v [B,Hkv,Lmax,D]")
    B, Hq, q_len, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("q and k/v disagree on batch or head_dim")
    lens = np.ascontiguousarray(np.asarray(cache_lens, dtype=np.int32))
    if lens.shape != (B,):
        raise ValueError("cache_lens must have shape [B]")
    return q, k, v, lens, (B, Hq, Hkv, D, q_len, Lmax, code)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected its arguments (rc={rc})")


def attention(q, k, v, cache_lens, scale, nthreads: int = 0, lib=None):
    """Plain definition: returns (out [B,Hq,q_len,D], lse [B,Hq,q_len]) in fp64."""
    lib = lib or load()
    q, k, v, lens, dims = _prep(q, k, v, cache_lens)
    B, Hq, Hkv, D, q_len, Lmax, code = dims
    out = np.empty((B, Hq, q_len, D), np.float64)
    lse = np.empty((B, Hq, q_len), np.float64)
    rc = lib.orc_attention(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(lens),
                           float(np.float32(scale)), _ptr(out), _ptr(lse), nthreads)
    _check(rc, "attention")
    return out, lse


def attention_split(q, k, v, cache_lens, scale, num_splits: int = 0, tile_len: int = 0,
                    slots: int | None = None, nthreads: int = 0, lib=None):
    """Split form.  Returns (out, lse, o_part, m_part, lse_part).

    ``num_splits > 0``: tile = ceil(L_b / num_splits) for each sequence.
    ``num_splits == 0``: fixed tile ``tile_len``.
    ``slots``: partial slots per row (default: the largest tile count).
    """
    lib = lib or load()
    q, k, v, lens, dims = _prep(q, k, v, cache_lens)
    B, Hq, Hkv, D, q_len, Lmax, code = dims
    if slots is None:
        counts = []
        for L in lens.tolist():
            T = -(-L // num_splits) if num_splits > 0 else tile_len
            T = max(T, 1)
            counts.append(-(-L // T))
        slots = max([1] + counts)
    out = np.empty((B, Hq, q_len, D), np.float64)
    lse = np.empty((B, Hq, q_len), np.float64)
    o_part = np.empty((B, Hq, q_len, slots, D), np.float64)
    m_part = np.empty((B, Hq, q_len, slots), np.float64)
    lse_part = np.empty((B, Hq, q_len, slots), np.float64)
    rc = lib.orc_attention_split(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(lens),
                                 float(np.float32(scale)), int(num_splits), int(tile_len),
                                 int(slots), _ptr(o_part), _ptr(m_part), _ptr(lse_part),
                                 _ptr(out), _ptr(lse), nthreads)
    _check(rc, "attention_split")
    return out, lse, o_part, m_part, lse_part


def span_ranges(cache_lens, num_kv_heads: int, spans: int, slots: int, piece_blocks: int = 16,
                block: int = 16):
    """Key ranges of the balanced-span split (the equal token bins of page
    "FlashDecoding算法原理与多GPU并行解码实战", variable-length section, with
    one bin per span instead of per device).

    Each (sequence b, KV head g) pair holds nb_b = ceil(L_b / block) blocks of
    ``block`` keys.  Lay the pairs with keys end to end on a line (sequence
    0's heads 0, 1, ..., then sequence 1's, ...), each taking
    ``piece_blocks`` positions for the fixed cost of a piece followed by its
    nb_b blocks, and cut the line every ``per`` positions, per =
    max(ceil(line length / spans), ceil(max nb_b / (slots - 1)), 1).  The
    blocks of one pair inside one cut are one piece; its pieces, in key
    order, are its slots 0, 1, ...: slot i of the pair is cut k0 + i, where
    k0 is the cut holding the pair's first block.  Returns (lo, hi, per):
    int32 arrays [B, Hkv, slots] of key ranges (lo == hi == 0: an empty
    slot) and the cut length in positions.
    """
    lens = [max(0, int(x)) for x in np.asarray(cache_lens).reshape(-1)]
    if slots < 2 or spans < 1:
        raise ValueError("spans need at least 2 slots and 1 span")
    nb = [-(-L // block) for L in lens]
    line = sum(num_kv_heads * (piece_blocks + n) for n in nb if n > 0)
    per = max(-(-line // spans), -(-max(nb + [0]) // (slots - 1)), 1)
    lo = np.zeros((len(lens), num_kv_heads, slots), np.int32)
    hi = np.zeros_like(lo)
    pos = 0  # line position of the current pair
    for b, L in enumerate(lens):
        if nb[b] == 0:
            continue
        for g in range(num_kv_heads):
            first = pos + piece_blocks  # line position of the pair's block 0
            first_cut = first // per
            for cut in range(first_cut, (first + nb[b] - 1) // per + 1):
                a = max(cut * per, first) - first
                e = min((cut + 1) * per, first + nb[b]) - first
                i = cut - first_cut
                if i >= slots:
                    raise AssertionError("a pair needs more slots than the rule allows")
                lo[b, g, i] = a * block
                hi[b, g, i] = min(e * block, L)
            pos = first + nb[b]
    return lo, hi, per


def attention_ranges(q, k, v, cache_lens, scale, lo, hi, nthreads: int = 0, lib=None):
    """Split form over explicit key ranges ``lo``/``hi`` [B, Hkv, S] per
    (sequence, KV head) and slot.  Returns (out, lse, o_part, m_part,
    lse_part); a slot whose range holds no visible key of a row has m = lse =
    -inf and o = 0 there."""
    lib = lib or load()
    q, k, v, lens, dims = _prep(q, k, v, cache_lens)
    B, Hq, Hkv, D, q_len, Lmax, code = dims
    lo = np.ascontiguousarray(lo, dtype=np.int32)
    hi = np.ascontiguousarray(hi, dtype=np.int32)
    if lo.shape != hi.shape or lo.ndim != 3 or lo.shape[:2] != (B, Hkv):
        raise ValueError("lo and hi must be [B, Hkv, S]")
    S = lo.shape[2]
    out = np.empty((B, Hq, q_len, D), np.float64)
    lse = np.empty((B, Hq, q_len), np.float64)
    o_part = np.empty((B, Hq, q_len, S, D), np.float64)
    m_part = np.empty((B, Hq, q_len, S), np.float64)
    lse_part = np.empty((B, Hq, q_len, S), np.float64)
    rc = lib.orc_attention_ranges(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(lens),
                                  float(np.float32(scale)), int(S), _ptr(lo), _ptr(hi),
                                  _ptr(o_part), _ptr(m_part), _ptr(lse_part), _ptr(out), _ptr(lse),
                                  nthreads)
    _check(rc, "attention_ranges")
    return out, lse, o_part, m_part, lse_part


def attention_sequential(q, k, v, cache_lens, scale, block: int = 256, nthreads: int = 0,
                         lib=None):
    """Running-rescaling form over fixed blocks of ``block`` keys."""
    lib = lib or load()
    q, k, v, lens, dims = _prep(q, k, v, cache_lens)
    B, Hq, Hkv, D, q_len, Lmax, code = dims
    out = np.empty((B, Hq, q_len, D), np.float64)
    lse = np.empty((B, Hq, q_len), np.float64)
    rc = lib.orc_attention_sequential(*dims, _ptr(q), _ptr(k), _ptr(v), _ptr(lens),
                                      float(np.float32(scale)), int(block), _ptr(out),
                                      _ptr(lse), nthreads)
    _check(rc, "attention_sequential")
    return out, lse


def merge_lse(o_part, lse_part, lib=None):
    """Merge partials o_part [..., S, D] with lse_part [..., S] into (out, lse)."""
    lib = lib or load()
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    S, D = o_part.shape[-2], o_part.shape[-1]
    lead = o_part.shape[:-2]
    if lse_part.shape != lead + (S,):
        raise ValueError("lse_part must be o_part's shape without the last axis")
    rows = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (D,), np.float64)
    lse = np.empty(lead, np.float64)
    rc = lib.orc_merge_lse(rows, S, D, _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse))
    _check(rc, "merge_lse")
    return out, lse


def gather_pages(pages, block_table, cache_lens, layout: str = "nhd"):
    """Contiguous ``[B, Hkv, Lmax, D]`` copy of a paged cache, key by key.

    ``pages``: ``[num_pages, page_size, Hkv, D]`` (layout "nhd", the page
    layout named in page "FlashDecoding算法原理与多GPU并行解码实战",
    deployment engineering details item 1) or ``[num_pages, Hkv, page_size, D]``
    ("hnd").  Key j of sequence b is row ``j % page_size`` of page
    ``block_table[b, j // page_size]``; ``Lmax = block_table.shape[1] *
    page_size``.  Keys at or past ``cache_lens[b]`` are left zero (the
    attention never reads them).
    """
    pages = np.asarray(pages)
    table = np.asarray(block_table)
    if layout == "nhd":
        _, P, H, D = pages.shape
    elif layout == "hnd":
        _, H, P, D = pages.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    B, max_pages = table.shape
    out = np.zeros((B, H, max_pages * P, D), pages.dtype)
    for b in range(B):
        for j in range(int(cache_lens[b])):
            page, row = int(table[b, j // P]), j % P
            out[b, :, j, :] = pages[page, row, :, :] if layout == "nhd" else pages[page, :, row, :]
    return out


def attention_paged(q, k_pages, v_pages, block_table, cache_lens, scale, layout: str = "nhd",
                    nthreads: int = 0, lib=None):
    """The plain definition over a paged cache: gather, then ``attention``."""
    lens = np.asarray(cache_lens, dtype=np.int32)
    k = gather_pages(k_pages, block_table, lens, layout)
    v = gather_pages(v_pages, block_table, lens, layout)
    return attention(q, k, v, lens, scale, nthreads=nthreads, lib=lib)


def fp8_e4m3_to_float(codes):
    """Values of OCP FP8 E4M3 ("e4m3fn") codes as float64, from the format's
    definition: sign bit 7, exponent bits 6:3 with bias 7, mantissa bits 2:0;
    exponent 0 is subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN; no
    infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _attention_codes(q, kf, vf, cache_lens, scale, k_scale, v_scale, nthreads, lib, what):
    """The plain definition over dequantised caches: kf/vf hold the code
    values (exact in float32); key = code * k_scale enters through the exact
    fp64 product scale * k_scale (scores are linear in the key), and v_scale
    multiplies the output (the output is linear in V)."""
    lib = lib or load()
    qf = np.ascontiguousarray(q)
    if qf.dtype == np.uint16:
        qf = (qf.astype(np.uint32) << 16).view(np.float32)
    qf, kf, vf, lens, dims = _prep(qf, np.ascontiguousarray(kf), np.ascontiguousarray(vf), cache_lens)
    B, Hq, Hkv, D, q_len, Lmax, code = dims
    out = np.empty((B, Hq, q_len, D), np.float64)
    lse = np.empty((B, Hq, q_len), np.float64)
    s = float(np.float32(scale)) * float(np.float32(k_scale))
    rc = lib.orc_attention(*dims, _ptr(qf), _ptr(kf), _ptr(vf), _ptr(lens), s, _ptr(out), _ptr(lse), nthreads)
    _check(rc, what)
    return out * float(np.float32(v_scale)), lse


def attention_fp8(q, k_codes, v_codes, cache_lens, scale, k_scale, v_scale, nthreads: int = 0, lib=None):
    """The plain definition over FP8 E4M3 caches: key = code * k_scale and
    value = code * v_scale (the dequantisation of page "FlashDecoding算法原理与
    多GPU并行解码实战", section on combining methods).  ``q`` holds bf16 bit
    patterns (uint16) or float32 values; ``k_codes``/``v_codes`` uint8 codes of
    shape [B, Hkv, Lmax, D].
    """
    kf = fp8_e4m3_to_float(k_codes).astype(np.float32)
    vf = fp8_e4m3_to_float(v_codes).astype(np.float32)
    return _attention_codes(q, kf, vf, cache_lens, scale, k_scale, v_scale, nthreads, lib, "attention_fp8")


def int8_to_float(codes):
    """Values of two's-complement INT8 codes as float64, from the encoding's
    definition: a byte c (0..255) stands for c - 256 when its bit 7 is set,
    else for c."""
    c = np.asarray(codes).view(np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def attention_int8(q, k_codes, v_codes, cache_lens, scale, k_scale, v_scale, nthreads: int = 0, lib=None):
    """The plain definition over INT8 caches (the other cache format of the
    same section): key = code * k_scale, value = code * v_scale, with int8
    (or uint8-viewed) codes of shape [B, Hkv, Lmax, D]; as attention_fp8."""
    kf = int8_to_float(k_codes).astype(np.float32)
    vf = int8_to_float(v_codes).astype(np.float32)
    return _attention_codes(q, kf, vf, cache_lens, scale, k_scale, v_scale, nthreads, lib, "attention_int8")