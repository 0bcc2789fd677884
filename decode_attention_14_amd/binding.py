"""Python binding of the C ABI in ``include/fd.h`` (ctypes; argument marshalling only).

torch supplies device memory and the stream: tensors are passed as raw device
pointers, and work is enqueued on ``torch.cuda.current_stream()`` of the input
device.  Every computation runs in the HIP kernels of ``libfd.so``; if the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FD_LIBRARY", os.path.join(_PKG, "libfd.so"))

FD_OK, FD_ERR_INVALID, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_ERR_DEVICE = 0, -1, -2, -3, -4
FD_F32, FD_BF16, FD_FP8_E4M3, FD_INT8 = 0, 1, 2, 3
FD_MAX_SPLITS = 256
FD_NOALLOC_SCRATCH_BYTES = 32 << 20

FD_PAGES_NHD, FD_PAGES_HND = 0, 1

EXPORTS = ("fd_plan_splits", "fd_workspace_bytes", "fd_decode_partials", "fd_combine_splits",
           "fd_decode_attention", "fd_decode_attention_noalloc", "fd_decode_attention_paged", "fd_decode_partials_paged",
           "fd_decode_attention_fp8", "fd_decode_partials_fp8", "fd_decode_attention_int8",
           "fd_decode_partials_int8", "fd_stream_read", "fd_status_string", "fd_last_error", "fd_version")


class FdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("max_cache_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class FdPlan(ctypes.Structure):
    _fields_ = [("tile_len", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("work_units", ctypes.c_int32),
                ("spans", ctypes.c_int32)]

    def __repr__(self):
        return (f"FdPlan(tile_len={self.tile_len}, max_splits={self.max_splits}, "
                f"workspace_bytes={self.workspace_bytes}, work_units={self.work_units}, spans={self.spans})")


class FdKvPages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class FdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load ``libfd.so`` (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    dims_p, plan_p = ctypes.POINTER(FdDims), ctypes.POINTER(FdPlan)
    lib.fd_plan_splits.argtypes = [dims_p, vp, i32, i32, plan_p, vp]
    lib.fd_plan_splits.restype = i32
    lib.fd_workspace_bytes.argtypes = [dims_p, i32]
    lib.fd_workspace_bytes.restype = u64
    lib.fd_decode_partials.argtypes = [dims_p, vp, vp, vp, vp, ctypes.c_float, i32, plan_p,
                                       vp, vp, vp, vp]
    lib.fd_decode_partials.restype = i32
    lib.fd_combine_splits.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp]
    lib.fd_combine_splits.restype = i32
    lib.fd_decode_attention.argtypes = [dims_p, vp, vp, vp, vp, ctypes.c_float, i32, plan_p,
                                        vp, u64, vp, vp, vp]
    lib.fd_decode_attention.restype = i32
    lib.fd_decode_attention_noalloc.argtypes = [dims_p, vp, vp, vp, vp, ctypes.c_float, i32, plan_p, vp, vp, vp]
    lib.fd_decode_attention_noalloc.restype = i32
    lib.fd_decode_attention_paged.argtypes = [dims_p, vp, vp, vp, ctypes.POINTER(FdKvPages), vp,
                                              ctypes.c_float, i32, plan_p, vp, u64, vp, vp, vp]
    lib.fd_decode_attention_paged.restype = i32
    lib.fd_decode_partials_paged.argtypes = [dims_p, vp, vp, vp, ctypes.POINTER(FdKvPages), vp,
                                             ctypes.c_float, i32, plan_p, vp, vp, vp, vp]
    lib.fd_decode_partials_paged.restype = i32
    pages_p, f32 = ctypes.POINTER(FdKvPages), ctypes.c_float
    lib.fd_decode_attention_fp8.argtypes = [dims_p, vp, vp, vp, pages_p, f32, f32, vp, f32, i32, plan_p,
                                            vp, u64, vp, vp, vp]
    lib.fd_decode_attention_fp8.restype = i32
    lib.fd_decode_partials_fp8.argtypes = [dims_p, vp, vp, vp, pages_p, f32, f32, vp, f32, i32, plan_p,
                                           vp, vp, vp, vp]
    lib.fd_decode_partials_fp8.restype = i32
    lib.fd_decode_attention_int8.argtypes = lib.fd_decode_attention_fp8.argtypes
    lib.fd_decode_attention_int8.restype = i32
    lib.fd_decode_partials_int8.argtypes = lib.fd_decode_partials_fp8.argtypes
    lib.fd_decode_partials_int8.restype = i32
    lib.fd_stream_read.argtypes = [vp, u64, i32, i32, vp, vp]
    lib.fd_stream_read.restype = i32
    lib.fd_status_string.argtypes = [i32]
    lib.fd_status_string.restype = ctypes.c_char_p
    lib.fd_last_error.argtypes = []
    lib.fd_last_error.restype = ctypes.c_char_p
    lib.fd_version.argtypes = []
    lib.fd_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def use_library(path: str):
    """Load the library build at ``path`` (same ABI, e.g. the workgroup-
    timeline diagnostic build) and route every later call of this module
    through it."""
    global _lib
    _lib = load_library(path)
    return _lib


def status_string(status: int) -> str:
    return load_library().fd_status_string(status).decode()


def _check(status: int):
    if status != FD_OK:
        raise FdError(status, load_library().fd_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return FD_BF16
    if t == torch.float32:
        return FD_F32
    raise FdError(FD_ERR_UNSUPPORTED, f"dtype {t} not supported (bfloat16 or float32)")


def make_dims(batch, num_q_heads, num_kv_heads, head_dim, q_len, max_cache_len, dtype) -> FdDims:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return FdDims(batch, num_q_heads, num_kv_heads, head_dim, q_len, max_cache_len, code)


def dims_of(q: torch.Tensor, k: torch.Tensor) -> FdDims:
    if q.dim() != 4 or k.dim() != 4:
        raise FdError(FD_ERR_INVALID, "q must be [B,Hq,q_len,D] and k_cache [B,Hkv,Lmax,D]")
    B, Hq, q_len, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D:
        raise FdError(FD_ERR_INVALID, f"q {tuple(q.shape)} and k_cache {tuple(k.shape)} disagree")
    return make_dims(B, Hq, Hkv, D, q_len, Lmax, q.dtype)


@dataclass
class Plan:
    plan: FdPlan
    splits_per_seq: list

    @property
    def tile_len(self):
        return self.plan.tile_len

    @property
    def max_splits(self):
        return self.plan.max_splits

    @property
    def workspace_bytes(self):
        return self.plan.workspace_bytes

    @property
    def spans(self):
        return self.plan.spans


def plan_splits(dims: FdDims, cache_lens_host, num_splits: int = 0, num_cus: int = 0) -> Plan:
    """Host-side split plan from host lengths (list, numpy array or CPU tensor)."""
    lib = load_library()
    lens = torch.as_tensor(cache_lens_host, dtype=torch.int32).cpu().contiguous()
    if lens.numel() != dims.batch:
        raise FdError(FD_ERR_INVALID, "cache_lens must have batch entries")
    splits = torch.zeros(max(dims.batch, 1), dtype=torch.int32)
    p = FdPlan()
    _check(lib.fd_plan_splits(ctypes.byref(dims), ctypes.c_void_p(lens.data_ptr()),
                              int(num_splits), int(num_cus), ctypes.byref(p),
                              ctypes.c_void_p(splits.data_ptr())))
    return Plan(p, splits[:dims.batch].tolist())


def plan_for(q: torch.Tensor, k: torch.Tensor, cache_lens_host, num_splits: int = 0,
             num_cus: int = 0) -> Plan:
    return plan_splits(dims_of(q, k), cache_lens_host, num_splits, num_cus)


def workspace_bytes(dims: FdDims, max_splits: int) -> int:
    return int(load_library().fd_workspace_bytes(ctypes.byref(dims), int(max_splits)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Device memory for a decode_attention workspace (contents irrelevant)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_inputs(q, k_cache, v_cache, cache_lens):
    if v_cache.shape != k_cache.shape:
        raise FdError(FD_ERR_INVALID, f"v_cache {tuple(v_cache.shape)} != k_cache {tuple(k_cache.shape)}")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise FdError(FD_ERR_INVALID, "q, k_cache and v_cache must share one dtype")
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (q.shape[0],):
        raise FdError(FD_ERR_INVALID, "cache_lens must be int32 of shape [B]")
    devs = {t.device for t in (q, k_cache, v_cache, cache_lens)}
    if len(devs) != 1:
        raise FdError(FD_ERR_INVALID, "all tensors must be on one device")


def _check_buffer(t, shape, dtype, name):
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise FdError(FD_ERR_INVALID, f"{name} must be {dtype} of shape {tuple(shape)}")


def _default_scale(D, scale):
    return float(1.0 / math.sqrt(D)) if scale is None else float(scale)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise FdError(FD_ERR_INVALID, "tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise FdError(FD_ERR_INVALID, "tensors must be contiguous")


def decode_attention(q, k_cache, v_cache, cache_lens, scale=None, num_splits: int = 0,
                     plan: Plan | FdPlan | None = None, out=None, lse=None, workspace=None):
    """Split-KV attention.  Returns (out, lse); allocates what is not given.

    q [B,Hq,q_len,D]; k_cache, v_cache [B,Hkv,Lmax,D]; cache_lens [B] int32 on
    the device.  ``num_splits > 0`` forces the split count; otherwise ``plan``
    (None: a single tile per sequence).
    """
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, cache_lens, out, lse, workspace)
    dims = dims_of(q, k_cache)
    _check_inputs(q, k_cache, v_cache, cache_lens)
    _check_buffer(out, q.shape, q.dtype, "out")
    _check_buffer(lse, q.shape[:3], torch.float32, "lse")
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws_bytes = workspace_bytes(dims, slots) if slots > 1 else 0
    if workspace is None and ws_bytes:
        workspace = new_workspace(ws_bytes, q.device)
    given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.fd_decode_attention(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(cache_lens), ctypes.c_float(_default_scale(q.shape[-1], scale)),
                                   int(num_splits), ctypes.byref(fp) if fp is not None else None,
                                   _ptr(workspace), given, _ptr(out), _ptr(lse),
                                   _stream(q.device)))
    return out, lse


def decode_attention_noalloc(q, k_cache, v_cache, cache_lens, scale=None, num_splits: int = 0,
                             plan: Plan | FdPlan | None = None, out=None, lse=None):
    """decode_attention through fd_decode_attention_noalloc: the library's
    static per-GPU scratch holds the partials (no workspace).  Returns
    (out, lse); out and lse are allocated here when not given."""
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, cache_lens, out, lse)
    dims = dims_of(q, k_cache)
    _check_inputs(q, k_cache, v_cache, cache_lens)
    _check_buffer(out, q.shape, q.dtype, "out")
    _check_buffer(lse, q.shape[:3], torch.float32, "lse")
    fp = plan.plan if isinstance(plan, Plan) else plan
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib.fd_decode_attention_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(cache_lens), ctypes.c_float(_default_scale(q.shape[-1], scale)),
                                           int(num_splits), ctypes.byref(fp) if fp is not None else None,
                                           _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def decode_partials(q, k_cache, v_cache, cache_lens, scale=None, num_splits: int = 0,
                    plan: Plan | FdPlan | None = None, o_part=None, m_part=None, lse_part=None):
    """First pass only.  Returns (o_part [B,Hq,q_len,S,D], m_part, lse_part [B,Hq,q_len,S])."""
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, cache_lens, o_part, m_part, lse_part)
    dims = dims_of(q, k_cache)
    _check_inputs(q, k_cache, v_cache, cache_lens)
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 0)
    if slots < 1:
        raise FdError(FD_ERR_INVALID, "decode_partials needs num_splits > 0 or a plan")
    B, Hq, T, D = q.shape
    _check_buffer(o_part, (B, Hq, T, slots, D), torch.float32, "o_part")
    _check_buffer(m_part, (B, Hq, T, slots), torch.float32, "m_part")
    _check_buffer(lse_part, (B, Hq, T, slots), torch.float32, "lse_part")
    if o_part is None:
        o_part = torch.empty(B, Hq, T, slots, D, dtype=torch.float32, device=q.device)
    if m_part is None:
        m_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    _check(lib.fd_decode_partials(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(cache_lens), ctypes.c_float(_default_scale(D, scale)),
                                  int(num_splits), ctypes.byref(fp) if fp is not None else None,
                                  _ptr(o_part), _ptr(m_part), _ptr(lse_part), _stream(q.device)))
    return o_part, m_part, lse_part


def combine(o_part, lse_part, out_dtype=torch.float32, out=None, lse=None, splits=None):
    """Second pass only: o_part [B,H,T,S,D], lse_part [B,H,T,S] fp32 -> (out, lse).

    ``splits``: optional int32 device tensor [B]; the rows of sequence b merge
    only their first splits[b] slots (None: all S)."""
    lib = load_library()
    _require_cuda(o_part, lse_part, out, lse, splits)
    if o_part.dim() != 5 or lse_part.shape != o_part.shape[:4]:
        raise FdError(FD_ERR_INVALID, "o_part must be [B,H,T,S,D] and lse_part [B,H,T,S]")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise FdError(FD_ERR_INVALID, "partials must be float32")
    B, H, T, S, D = o_part.shape
    if splits is not None and (splits.dtype != torch.int32 or tuple(splits.shape) != (B,)):
        raise FdError(FD_ERR_INVALID, "splits must be int32 of shape [B]")
    _check_buffer(out, (B, H, T, D), out.dtype if out is not None else out_dtype, "out")
    _check_buffer(lse, (B, H, T), torch.float32, "lse")
    if out is None:
        out = torch.empty(B, H, T, D, dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty(B, H, T, dtype=torch.float32, device=o_part.device)
    _check(lib.fd_combine_splits(B, H, T, D, S, _ptr(o_part), _ptr(lse_part), _ptr(splits),
                                 _dtype_code(out.dtype), _ptr(out), _ptr(lse),
                                 _stream(o_part.device)))
    return out, lse


def stream_read(buf: torch.Tensor, nbytes: int | None = None, workgroups: int = 0, sink=None, offset: int = 0,
                pattern: int = 0):
    """Measurement aid: one streaming read of ``nbytes`` bytes of ``buf``
    from byte ``offset`` on (all of it by default) by the library's read
    kernel, enqueued on the current stream; ``pattern`` 0 strides over the
    grid, 1 gives each workgroup a contiguous range.  Returns the 4-byte
    sink tensor."""
    lib = load_library()
    _require_cuda(buf, sink)
    total = buf.numel() * buf.element_size()
    n = total - offset if nbytes is None else int(nbytes)
    if offset < 0 or n < 0 or offset + n > total:
        raise FdError(FD_ERR_INVALID, "read range outside the buffer")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(lib.fd_stream_read(ctypes.c_void_p(buf.data_ptr() + offset), n, int(workgroups), int(pattern), _ptr(sink),
                              _stream(buf.device)))
    return sink


_LAYOUTS = {"nhd": FD_PAGES_NHD, "hnd": FD_PAGES_HND}


def paged_dims(q: torch.Tensor, k_pages: torch.Tensor, block_table: torch.Tensor, layout: str = "nhd"):
    """(dims, page_size, num_kv_heads) of a paged call.

    k_pages is [num_pages, page_size, Hkv, D] ("nhd") or [num_pages, Hkv, page_size, D]
    ("hnd"); block_table [B, max_pages_per_seq] int32.
    """
    if layout not in _LAYOUTS:
        raise FdError(FD_ERR_UNSUPPORTED, f"page layout {layout!r} unknown (nhd or hnd)")
    if q.dim() != 4 or k_pages.dim() != 4 or block_table.dim() != 2:
        raise FdError(FD_ERR_INVALID, "q must be [B,Hq,q_len,D], k_pages 4-d and block_table [B, pages]")
    B, Hq, q_len, D = q.shape
    if layout == "nhd":
        _, P, Hkv, Dk = k_pages.shape
    else:
        _, Hkv, P, Dk = k_pages.shape
    if Dk != D or block_table.shape[0] != B:
        raise FdError(FD_ERR_INVALID, f"q {tuple(q.shape)}, k_pages {tuple(k_pages.shape)} and "
                                      f"block_table {tuple(block_table.shape)} disagree")
    return make_dims(B, Hq, Hkv, D, q_len, block_table.shape[1] * P, q.dtype), P


def _paged_args(q, k_pages, v_pages, block_table, cache_lens, layout):
    dims, P = paged_dims(q, k_pages, block_table, layout)
    if v_pages.shape != k_pages.shape:
        raise FdError(FD_ERR_INVALID, f"v_pages {tuple(v_pages.shape)} != k_pages {tuple(k_pages.shape)}")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise FdError(FD_ERR_INVALID, "q, k_pages and v_pages must share one dtype")
    if block_table.dtype != torch.int32:
        raise FdError(FD_ERR_INVALID, "block_table must be int32")
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (q.shape[0],):
        raise FdError(FD_ERR_INVALID, "cache_lens must be int32 of shape [B]")
    if len({t.device for t in (q, k_pages, v_pages, block_table, cache_lens)}) != 1:
        raise FdError(FD_ERR_INVALID, "all tensors must be on one device")
    pages = FdKvPages(block_table.data_ptr(), block_table.shape[1], P, k_pages.shape[0], _LAYOUTS[layout])
    return dims, pages


def decode_attention_paged(q, k_pages, v_pages, block_table, cache_lens, layout: str = "nhd",
                           scale=None, num_splits: int = 0, plan: Plan | FdPlan | None = None,
                           out=None, lse=None, workspace=None):
    """Split-KV attention over a paged K/V cache.  Returns (out, lse).

    k_pages, v_pages: [num_pages, page_size, Hkv, D] (layout "nhd") or
    [num_pages, Hkv, page_size, D] ("hnd"); block_table [B, max_pages_per_seq]
    int32 on the device; key j of sequence b is row j % page_size of page
    block_table[b, j // page_size].  Other arguments as decode_attention; a
    plan comes from plan_splits(paged_dims(...)[0], lengths).
    """
    lib = load_library()
    _require_cuda(q, k_pages, v_pages, block_table, cache_lens, out, lse, workspace)
    dims, pages = _paged_args(q, k_pages, v_pages, block_table, cache_lens, layout)
    _check_buffer(out, q.shape, q.dtype, "out")
    _check_buffer(lse, q.shape[:3], torch.float32, "lse")
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws_bytes = workspace_bytes(dims, slots) if slots > 1 else 0
    if workspace is None and ws_bytes:
        workspace = new_workspace(ws_bytes, q.device)
    given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.fd_decode_attention_paged(ctypes.byref(dims), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                         ctypes.byref(pages), _ptr(cache_lens),
                                         ctypes.c_float(_default_scale(q.shape[-1], scale)),
                                         int(num_splits), ctypes.byref(fp) if fp is not None else None,
                                         _ptr(workspace), given, _ptr(out), _ptr(lse),
                                         _stream(q.device)))
    return out, lse


def decode_partials_paged(q, k_pages, v_pages, block_table, cache_lens, layout: str = "nhd", scale=None,
                          num_splits: int = 0, plan: Plan | FdPlan | None = None, o_part=None, m_part=None,
                          lse_part=None):
    """First pass only, over a paged cache: (o_part, m_part, lse_part) as decode_partials."""
    lib = load_library()
    _require_cuda(q, k_pages, v_pages, block_table, cache_lens, o_part, m_part, lse_part)
    dims, pages = _paged_args(q, k_pages, v_pages, block_table, cache_lens, layout)
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 0)
    if slots < 1:
        raise FdError(FD_ERR_INVALID, "decode_partials_paged needs num_splits > 0 or a plan")
    B, Hq, T, D = q.shape
    _check_buffer(o_part, (B, Hq, T, slots, D), torch.float32, "o_part")
    _check_buffer(m_part, (B, Hq, T, slots), torch.float32, "m_part")
    _check_buffer(lse_part, (B, Hq, T, slots), torch.float32, "lse_part")
    if o_part is None:
        o_part = torch.empty(B, Hq, T, slots, D, dtype=torch.float32, device=q.device)
    if m_part is None:
        m_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    _check(lib.fd_decode_partials_paged(ctypes.byref(dims), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                        ctypes.byref(pages), _ptr(cache_lens),
                                        ctypes.c_float(_default_scale(D, scale)), int(num_splits),
                                        ctypes.byref(fp) if fp is not None else None, _ptr(o_part),
                                        _ptr(m_part), _ptr(lse_part), _stream(q.device)))
    return o_part, m_part, lse_part


_CODE_DTYPES = {"fp8": torch.uint8, "int8": torch.int8}


def _code_call_args(fmt, q, k_cache, v_cache, cache_lens, block_table, layout):
    """(dims, pages or None) of a call over one-byte codes: uint8 E4M3 codes
    ("fp8") or int8 codes ("int8")."""
    want = _CODE_DTYPES[fmt]
    if k_cache.dtype != want or v_cache.dtype != want:
        raise FdError(FD_ERR_INVALID, f"{fmt} caches are passed as {want} tensors of codes")
    if v_cache.shape != k_cache.shape:
        raise FdError(FD_ERR_INVALID, f"v_cache {tuple(v_cache.shape)} != k_cache {tuple(k_cache.shape)}")
    if q.dtype != torch.bfloat16:
        raise FdError(FD_ERR_UNSUPPORTED, f"{fmt} caches need a bf16 q")
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (q.shape[0],):
        raise FdError(FD_ERR_INVALID, "cache_lens must be int32 of shape [B]")
    if block_table is None:
        dims = dims_of(q, k_cache)
        dims.dtype = FD_BF16
        return dims, None
    if block_table.dtype != torch.int32:
        raise FdError(FD_ERR_INVALID, "block_table must be int32")
    dims, P = paged_dims(q, k_cache, block_table, layout)
    dims.dtype = FD_BF16
    return dims, FdKvPages(block_table.data_ptr(), block_table.shape[1], P, k_cache.shape[0], _LAYOUTS[layout])


def _codes_attention(fmt, q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                     num_splits, plan, out, lse, workspace):
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, cache_lens, block_table, out, lse, workspace)
    dims, pages = _code_call_args(fmt, q, k_cache, v_cache, cache_lens, block_table, layout)
    _check_buffer(out, q.shape, q.dtype, "out")
    _check_buffer(lse, q.shape[:3], torch.float32, "lse")
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws_bytes = workspace_bytes(dims, slots) if slots > 1 else 0
    if workspace is None and ws_bytes:
        workspace = new_workspace(ws_bytes, q.device)
    given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = lib.fd_decode_attention_fp8 if fmt == "fp8" else lib.fd_decode_attention_int8
    _check(fn(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
              ctypes.byref(pages) if pages is not None else None,
              ctypes.c_float(k_scale), ctypes.c_float(v_scale), _ptr(cache_lens),
              ctypes.c_float(_default_scale(q.shape[-1], scale)), int(num_splits),
              ctypes.byref(fp) if fp is not None else None, _ptr(workspace), given,
              _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def _codes_partials(fmt, q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                    num_splits, plan, o_part, m_part, lse_part):
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, cache_lens, block_table, o_part, m_part, lse_part)
    dims, pages = _code_call_args(fmt, q, k_cache, v_cache, cache_lens, block_table, layout)
    fp = plan.plan if isinstance(plan, Plan) else plan
    slots = num_splits if num_splits > 0 else (fp.max_splits if fp is not None else 0)
    if slots < 1:
        raise FdError(FD_ERR_INVALID, f"decode_partials_{fmt} needs num_splits > 0 or a plan")
    B, Hq, T, D = q.shape
    _check_buffer(o_part, (B, Hq, T, slots, D), torch.float32, "o_part")
    _check_buffer(m_part, (B, Hq, T, slots), torch.float32, "m_part")
    _check_buffer(lse_part, (B, Hq, T, slots), torch.float32, "lse_part")
    if o_part is None:
        o_part = torch.empty(B, Hq, T, slots, D, dtype=torch.float32, device=q.device)
    if m_part is None:
        m_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty(B, Hq, T, slots, dtype=torch.float32, device=q.device)
    fn = lib.fd_decode_partials_fp8 if fmt == "fp8" else lib.fd_decode_partials_int8
    _check(fn(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
              ctypes.byref(pages) if pages is not None else None,
              ctypes.c_float(k_scale), ctypes.c_float(v_scale), _ptr(cache_lens),
              ctypes.c_float(_default_scale(D, scale)), int(num_splits),
              ctypes.byref(fp) if fp is not None else None, _ptr(o_part), _ptr(m_part),
              _ptr(lse_part), _stream(q.device)))
    return o_part, m_part, lse_part


def decode_attention_fp8(q, k_cache, v_cache, cache_lens, k_scale: float, v_scale: float, block_table=None,
                         layout: str = "nhd", scale=None, num_splits: int = 0, plan: Plan | FdPlan | None = None,
                         out=None, lse=None, workspace=None):
    """Split-KV attention over FP8 E4M3 caches (uint8 codes; key = code * k_scale,
    value = code * v_scale).  Contiguous [B,Hkv,Lmax,D] caches, or pages with a
    block table as in decode_attention_paged.  q and out are bf16.  Returns (out, lse)."""
    return _codes_attention("fp8", q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                            num_splits, plan, out, lse, workspace)


def decode_partials_fp8(q, k_cache, v_cache, cache_lens, k_scale: float, v_scale: float, block_table=None,
                        layout: str = "nhd", scale=None, num_splits: int = 0, plan: Plan | FdPlan | None = None,
                        o_part=None, m_part=None, lse_part=None):
    """First pass only over FP8 caches: (o_part, m_part, lse_part) as decode_partials."""
    return _codes_partials("fp8", q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                           num_splits, plan, o_part, m_part, lse_part)


def decode_attention_int8(q, k_cache, v_cache, cache_lens, k_scale: float, v_scale: float, block_table=None,
                          layout: str = "nhd", scale=None, num_splits: int = 0, plan: Plan | FdPlan | None = None,
                          out=None, lse=None, workspace=None):
    """Split-KV attention over INT8 caches (int8 codes; key = code * k_scale,
    value = code * v_scale), otherwise as decode_attention_fp8.  Returns (out, lse)."""
    return _codes_attention("int8", q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                            num_splits, plan, out, lse, workspace)


def decode_partials_int8(q, k_cache, v_cache, cache_lens, k_scale: float, v_scale: float, block_table=None,
                         layout: str = "nhd", scale=None, num_splits: int = 0, plan: Plan | FdPlan | None = None,
                         o_part=None, m_part=None, lse_part=None):
    """First pass only over INT8 caches: (o_part, m_part, lse_part) as decode_partials."""
    return _codes_partials("int8", q, k_cache, v_cache, cache_lens, k_scale, v_scale, block_table, layout, scale,
                           num_splits, plan, o_part, m_part, lse_part)
