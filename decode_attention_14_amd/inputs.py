"""Seeded synthetic inputs for split-KV decode attention.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic.  Both the GPU path and the CPU oracle are fed from it.

Recipe (the same for every workload):
  * ``numpy.random.Generator(PCG64(seed))``;
  * draws in the order q, k, v, then the cache lengths;
  * q, k, v are ``standard_normal`` in float32, then rounded once to bf16
    (round-to-nearest-even, torch's CPU conversion) when the workload is bf16;
  * variable lengths are integers drawn uniformly from [lo, hi] inclusive.
Large tensors are drawn in slices of at most 2**26 values so host memory stays
bounded; the values equal those of one big draw from the same generator.

The workloads are the attention shapes of the pages' serving examples (a
Llama-3-8B-shaped layer at 32k context, a 70B-shaped batched layer with mixed
lengths, a long-context batch and one chunked-prefill chunk); N(0, 1) values
stand in for activations of trained models, which are not used here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_len: int
    max_cache_len: int
    dtype: str                      # "f32" or "bf16"
    seed: int
    cache_len: int | None = None    # fixed length for every sequence
    len_range: tuple | None = None  # (lo, hi) inclusive uniform lengths
    num_splits: int = 0             # forced split count (0: planner)
    notes: str = ""

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim) as the fp32 value the kernels receive."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("mha_tiny_1k", 1, 8, 8, 64, 1, 1024, "f32", 14001, cache_len=1024,
                 num_splits=4, notes="tiny MHA decode, 4 splits of 256 keys"),
        Workload("gqa_32k", 1, 32, 8, 128, 1, 32768, "bf16", 14002, cache_len=32768,
                 notes="Llama-3-8B-shaped GQA decode at 32k context"),
        Workload("varlen_b32", 32, 64, 8, 128, 1, 8192, "bf16", 14003, len_range=(512, 8192),
                 notes="70B-layer-shaped batched decode, lengths U[512, 8192]"),
        Workload("gqa_128k_b4", 4, 32, 8, 128, 1, 131072, "bf16", 14004, cache_len=131072,
                 notes="long-context GQA decode, 4 x 128k"),
        Workload("prefill_chunk_512", 1, 32, 8, 128, 512, 8192, "bf16", 14005, cache_len=8192,
                 notes="chunked-prefill chunk: 512 queries over 7680 cached + 512 new keys"),
        Workload("verify_q4_32k", 1, 32, 8, 128, 4, 32768, "bf16", 14006, cache_len=32768,
                 notes="speculative-decoding verification: 4 draft tokens (causal) over a 32k cache"),
    ]
}


def _normal(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    return out.reshape(shape)


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(batch, num_q_heads, num_kv_heads, head_dim, q_len, max_cache_len, dtype, seed,
                cache_len=None, len_range=None, cache_lens=None):
    """Draw (q, k, v, cache_lens) as CPU tensors.

    q ``[B, Hq, q_len, D]``, k and v ``[B, Hkv, Lmax, D]`` in ``dtype``
    ("f32" or "bf16"), cache_lens ``[B]`` int32.  Lengths come from
    ``cache_lens`` if given, else ``cache_len`` for every sequence, else a
    uniform draw from ``len_range``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _to_dtype(_normal(rng, (batch, num_q_heads, q_len, head_dim)), dtype)
    k = _to_dtype(_normal(rng, (batch, num_kv_heads, max_cache_len, head_dim)), dtype)
    v = _to_dtype(_normal(rng, (batch, num_kv_heads, max_cache_len, head_dim)), dtype)
    if cache_lens is not None:
        lens = np.asarray(cache_lens, dtype=np.int32)
    elif cache_len is not None:
        lens = np.full(batch, cache_len, np.int32)
    elif len_range is not None:
        lo, hi = len_range
        lens = rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    else:
        lens = np.full(batch, max_cache_len, np.int32)
    return q, k, v, torch.from_numpy(lens)


def workload_inputs(w: Workload):
    return make_inputs(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.q_len,
                       w.max_cache_len, w.dtype, w.seed, cache_len=w.cache_len,
                       len_range=w.len_range)


def as_oracle_array(t: torch.Tensor) -> np.ndarray:
    """Exact stored values for the oracle: float32 as is, bf16 as raw uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass(frozen=True)
class PagedCache:
    """A paged K/V cache built from contiguous caches (CPU tensors).

    ``k_pages``/``v_pages``: ``[num_pages, page_size, Hkv, D]`` ("nhd") or
    ``[num_pages, Hkv, page_size, D]`` ("hnd"); ``block_table`` ``[B, Lmax /
    page_size]`` int32, -1 where a sequence has no page.
    """
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor
    page_size: int
    layout: str


def paginate(k: torch.Tensor, v: torch.Tensor, cache_lens, page_size: int, layout: str = "nhd",
             seed: int = 0, spare_pages: int = 3) -> PagedCache:
    """Scatter contiguous caches ``[B, Hkv, Lmax, D]`` into a shuffled page pool.

    Sequence b gets ceil(L_b / page_size) pages; page ids are a seeded random
    permutation of the pool (``Generator(PCG64(seed)).permutation``), which
    also holds ``spare_pages`` pages no sequence uses.  Rows of a page at or
    past L_b and every spare page are filled with NaN (for uint8 FP8 codes,
    0x7F: the E4M3 NaN), so a kernel that reads them cannot go unnoticed;
    INT8 codes have no NaN, so their pools get 127, the largest code, which
    takes over the softmax of every query whose elements sum above zero.
    Data movement only.
    """
    if layout not in ("nhd", "hnd"):
        raise ValueError(f"unknown layout {layout!r}")
    B, H, Lmax, D = k.shape
    if Lmax % page_size:
        raise ValueError("Lmax must be a multiple of page_size")
    lens = [int(x) for x in torch.as_tensor(cache_lens).tolist()]
    counts = [-(-L // page_size) for L in lens]
    num_pages = sum(counts) + spare_pages
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(num_pages)
    table = torch.full((B, Lmax // page_size), -1, dtype=torch.int32)
    shape = (num_pages, page_size, H, D) if layout == "nhd" else (num_pages, H, page_size, D)
    fill = {torch.uint8: 0x7F, torch.int8: 127}.get(k.dtype, float("nan"))  # uint8: the E4M3 NaN code
    kp = torch.full(shape, fill, dtype=k.dtype)
    vp = torch.full(shape, fill, dtype=v.dtype)
    nxt = 0
    for b in range(B):
        for i in range(counts[b]):
            pid = int(perm[nxt])
            nxt += 1
            table[b, i] = pid
            lo, hi = i * page_size, min(lens[b], (i + 1) * page_size)
            src_k = k[b, :, lo:hi, :]  # [H, rows, D]
            src_v = v[b, :, lo:hi, :]
            if layout == "nhd":
                kp[pid, : hi - lo] = src_k.permute(1, 0, 2)
                vp[pid, : hi - lo] = src_v.permute(1, 0, 2)
            else:
                kp[pid, :, : hi - lo] = src_k
                vp[pid, :, : hi - lo] = src_v
    return PagedCache(kp, vp, table, page_size, layout)


def quantize_fp8(t: torch.Tensor, scale: float) -> torch.Tensor:
    """OCP FP8 E4M3 codes (uint8) of ``t / scale``, rounded to nearest even by
    torch's float8_e4m3fn conversion; |t / scale| must stay within 448."""
    x = t.float() / float(np.float32(scale))
    if float(x.abs().max()) > 448.0:
        raise ValueError("values exceed the E4M3 range at this scale")
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_int8(t: torch.Tensor, scale: float) -> torch.Tensor:
    """Symmetric INT8 codes of ``t / scale``: rounded to nearest even, then
    clamped to [-127, 127]."""
    x = torch.round(t.float() / float(np.float32(scale)))
    return x.clamp_(-127, 127).to(torch.int8)


def int8_scale_for(t: torch.Tensor) -> float:
    """Per-tensor scale mapping the largest |value| to 127, as an fp32 value."""
    return float(np.float32(float(t.float().abs().max()) / 127.0))


def fp8_scale_for(t: torch.Tensor) -> float:
    """Per-tensor scale mapping the largest |value| to 240 (headroom below the
    E4M3 maximum of 448), as an fp32 value."""
    return float(np.float32(float(t.float().abs().max()) / 240.0))
