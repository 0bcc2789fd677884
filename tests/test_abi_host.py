"""Host-side checks of the C ABI: the library loads, exports what the header
declares, the planner's properties hold, and malformed calls are rejected
before anything is enqueued.  No GPU is needed: every call here either is
host-only (the planner) or fails validation before any HIP call.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fd.h")

# Non-null, 256-byte aligned fake addresses.  Used only in calls that must fail
# validation; nothing ever dereferences them.
FAKE = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    return fd.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(fd.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_timeline_diagnostic_only_in_its_own_build(lib):
    """The workgroup-timeline diagnostic (FD_WG_TIMELINE=1) is a separate
    build with the same ABI plus fd_debug_timeline and fd_debug_chunk_timeline;
    libfd.so has none of it."""
    assert not hasattr(lib, "fd_debug_timeline")
    assert not hasattr(lib, "fd_debug_chunk_timeline")
    from decode_attention_14_amd.build import TIMELINE_LIB
    if not os.path.exists(TIMELINE_LIB):
        pytest.skip("the timeline build is made by __graft_entry__.build()")
    tl = ctypes.CDLL(TIMELINE_LIB)
    for name in fd.EXPORTS + ("fd_debug_timeline", "fd_debug_chunk_timeline"):
        assert hasattr(tl, name), name


def test_version_and_status_strings(lib):
    assert lib.fd_version() >= 100
    assert fd.status_string(fd.FD_OK) == "FD_OK"
    assert fd.status_string(fd.FD_ERR_WORKSPACE) == "FD_ERR_WORKSPACE"
    assert fd.status_string(-99) == "FD_STATUS_UNKNOWN"


def dims(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=32768, dt=fd.FD_BF16):
    return fd.make_dims(B, Hq, Hkv, D, T, Lmax, dt)


def tiles_of(L, tile_len, num_splits, slots):
    """The tile boundaries the ABI documents for one sequence."""
    T = tile_len if tile_len > 0 else -(-L // num_splits)
    T = max(T, 1)
    S = min(-(-L // T), slots)
    return [(s * T, L if s == S - 1 else min(L, (s + 1) * T)) for s in range(S)]


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_planner_on_workloads(name):
    w = WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    if w.len_range:
        lens = rng.integers(w.len_range[0], w.len_range[1] + 1, size=w.batch).tolist()
    else:
        lens = [w.cache_len] * w.batch
    d = fd.make_dims(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.q_len, w.max_cache_len,
                     fd.FD_BF16 if w.dtype == "bf16" else fd.FD_F32)
    p = fd.plan_splits(d, lens, num_splits=w.num_splits, num_cus=256)
    assert 1 <= p.max_splits <= fd.FD_MAX_SPLITS
    if w.num_splits:
        assert p.tile_len == 0 and p.max_splits == w.num_splits
    else:
        assert p.tile_len % 64 == 0
        # at least 256 keys, at most the longest sequence (rounded to 64)
        assert 256 <= p.tile_len <= max(256, -(-max(lens) // 64) * 64)
        # about one work unit per compute unit for equal lengths, four for
        # mixed ones: each (sequence, KV head, row block) adds at most one
        # unit beyond an even share
        rows = w.num_q_heads // w.num_kv_heads * w.q_len
        row_blocks = 1 if rows <= 32 else -(-rows // 128)
        lanes = w.num_kv_heads * row_blocks
        per_cu = 1 if min(lens) == max(lens) else 4
        assert p.plan.work_units <= per_cu * 256 + w.batch * lanes
    for L, S in zip(lens, p.splits_per_seq):
        t = tiles_of(L, p.tile_len, w.num_splits, p.max_splits)
        assert len(t) == S
        # exact, ordered partition of [0, L)
        assert t[0][0] == 0 and t[-1][1] == L
        assert all(a[1] == b[0] for a, b in zip(t, t[1:]))
        assert all(hi > lo for lo, hi in t)
    if p.max_splits > 1:
        assert p.workspace_bytes == fd.workspace_bytes(d, p.max_splits) > 0
    else:
        assert p.workspace_bytes == 0


def test_planner_headline_fills_the_chip():
    p = fd.plan_splits(dims(), [32768], num_cus=256)
    assert p.tile_len == 1024 and p.max_splits == 32
    assert p.plan.work_units == 8 * 32  # KV heads x tiles: one per CU


def test_planner_short_and_empty_sequences():
    p = fd.plan_splits(dims(B=4), [0, 1, 255, 256], num_cus=256)
    assert p.splits_per_seq == [0, 1, 1, 1]
    assert p.max_splits == 1 and p.workspace_bytes == 0


def test_planner_caps_splits_for_long_contexts():
    d = dims(B=1, Lmax=1 << 20)
    p = fd.plan_splits(d, [1 << 20], num_cus=256)
    assert p.max_splits <= fd.FD_MAX_SPLITS
    assert p.tile_len * p.max_splits >= 1 << 20


def test_planner_forced_counts_follow_ceil_rule():
    d = dims(B=5, Lmax=100)
    p = fd.plan_splits(d, [9, 0, 1, 100, 7], num_splits=4, num_cus=256)
    # ceil(L / ceil(L / 4)): 9 keys in chunks of 3 -> 3 tiles; 7 in chunks of 2 -> 4
    assert p.splits_per_seq == [3, 0, 1, 4, 4]
    assert p.max_splits == 4 and p.tile_len == 0


def test_planner_varlen_balances_units():
    w = WORKLOADS["varlen_b32"]
    rng = np.random.Generator(np.random.PCG64(3))
    lens = rng.integers(512, 8193, size=32).tolist()
    d = fd.make_dims(32, 64, 8, 128, 1, 8192, fd.FD_BF16)
    p = fd.plan_splits(d, lens, num_cus=256)
    tiles = [hi - lo for L in lens for lo, hi in tiles_of(L, p.tile_len, 0, p.max_splits)]
    assert max(tiles) <= p.tile_len
    assert p.plan.work_units == 8 * len(tiles)
    assert p.plan.work_units >= 4 * 256  # four units per CU for mixed lengths
    # the tile is the even share of four units per CU, rounded up to 64 keys
    assert p.tile_len == -(-(-(-sum(lens) * 8 // 1024)) // 64) * 64


@pytest.mark.parametrize("bad,status", [
    (dict(Hq=30, Hkv=8), fd.FD_ERR_INVALID),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(T=0), fd.FD_ERR_INVALID),
    (dict(dt=7), fd.FD_ERR_UNSUPPORTED),
    (dict(B=-1), fd.FD_ERR_INVALID),
    (dict(Lmax=-5), fd.FD_ERR_INVALID),
])
def test_planner_rejects_bad_dims(lib, bad, status):
    args = dict(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=64, dt=fd.FD_BF16)
    args.update(bad)
    d = dims(**args)
    lens = (ctypes.c_int32 * 1)(16)
    p = fd.FdPlan()
    assert lib.fd_plan_splits(ctypes.byref(d), lens, 0, 256, ctypes.byref(p), None) == status
    assert lib.fd_last_error().decode()


def test_planner_rejects_bad_lengths_and_counts(lib):
    d = dims(B=2, Lmax=64)
    p = fd.FdPlan()
    for lens, ns, cus in [((5, 65), 0, 256), ((-1, 3), 0, 256), ((5, 5), 257, 256),
                          ((5, 5), -1, 256), ((5, 5), 0, -1)]:
        arr = (ctypes.c_int32 * 2)(*lens)
        rc = lib.fd_plan_splits(ctypes.byref(d), arr, ns, cus, ctypes.byref(p), None)
        assert rc == fd.FD_ERR_INVALID, (lens, ns, cus)


def call_decode(lib, d, ptrs=None, num_splits=0, plan=None, ws=None, ws_bytes=0, out=None):
    q, k, v, lens, o, lse = ptrs or FAKE[:6]
    return lib.fd_decode_attention(ctypes.byref(d), q, k, v, lens, ctypes.c_float(0.1), num_splits,
                                   ctypes.byref(plan) if plan is not None else None, ws, ws_bytes,
                                   o if out is None else out, lse, None)


@pytest.mark.parametrize("bad,status", [
    (dict(Hq=12, Hkv=8), fd.FD_ERR_INVALID),
    (dict(D=256), fd.FD_ERR_UNSUPPORTED),
    (dict(T=0), fd.FD_ERR_INVALID),
    (dict(dt=3), fd.FD_ERR_UNSUPPORTED),
    (dict(B=70000), fd.FD_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_dims(lib, bad, status):
    args = dict(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=64, dt=fd.FD_BF16)
    args.update(bad)
    assert call_decode(lib, dims(**args)) == status


def test_decode_rejects_null_and_misaligned(lib):
    d = dims(Lmax=64)
    q, k, v, lens, o, lse = FAKE[:6]
    assert call_decode(lib, d, (None, k, v, lens, o, lse)) == fd.FD_ERR_INVALID
    assert call_decode(lib, d, (q, k, v, None, o, lse)) == fd.FD_ERR_INVALID
    assert call_decode(lib, d, (q, k, v, lens, None, lse)) == fd.FD_ERR_INVALID
    odd = ctypes.c_void_p(0x100008)
    assert call_decode(lib, d, (odd, k, v, lens, o, lse)) == fd.FD_ERR_INVALID
    assert call_decode(lib, d, (q, k, v, lens, odd, lse)) == fd.FD_ERR_INVALID
    assert call_decode(lib, d, (q, k, v, lens, o, ctypes.c_void_p(0x100002))) == fd.FD_ERR_INVALID
    assert "aligned" in lib.fd_last_error().decode()


def test_decode_rejects_missing_or_small_workspace(lib):
    d = dims(Lmax=64)
    assert call_decode(lib, d, num_splits=4) == fd.FD_ERR_WORKSPACE
    need = lib.fd_workspace_bytes(ctypes.byref(d), 4)
    assert need > 0
    assert call_decode(lib, d, num_splits=4, ws=FAKE[6], ws_bytes=need - 1) == fd.FD_ERR_WORKSPACE
    assert "workspace" in lib.fd_last_error().decode()
    # a misaligned workspace of the right size is rejected too
    assert call_decode(lib, d, num_splits=4, ws=ctypes.c_void_p(0x100010),
                       ws_bytes=need) == fd.FD_ERR_INVALID


def test_decode_rejects_bad_split_arguments(lib):
    d = dims(Lmax=64)
    assert call_decode(lib, d, num_splits=257) == fd.FD_ERR_INVALID
    assert call_decode(lib, d, num_splits=-2) == fd.FD_ERR_INVALID
    bad = fd.FdPlan(tile_len=0, max_splits=4)
    assert call_decode(lib, d, plan=bad) == fd.FD_ERR_INVALID
    bad = fd.FdPlan(tile_len=256, max_splits=300)
    assert call_decode(lib, d, plan=bad) == fd.FD_ERR_INVALID
    bad = fd.FdPlan(tile_len=256, max_splits=4, spans=-1)
    assert call_decode(lib, d, plan=bad) == fd.FD_ERR_INVALID
    bad = fd.FdPlan(tile_len=256, max_splits=4, spans=(1 << 20) + 1)
    assert call_decode(lib, d, plan=bad) == fd.FD_ERR_INVALID


def test_planner_asks_for_spans_only_past_one_round_of_tiles():
    """Mixed lengths with more tiles than two per compute unit get balanced
    spans (two per unit) and enough slots for them; equal lengths, small
    batches, fp32 and long chunks keep tiles."""
    rng = np.random.Generator(np.random.PCG64(3))
    lens = rng.integers(512, 8193, size=32).tolist()
    d = fd.make_dims(32, 64, 8, 128, 1, 8192, fd.FD_BF16)
    p = fd.plan_splits(d, lens, num_cus=256)
    assert p.spans == 512 and p.plan.work_units > 512
    # a pair of the longest sequence fits its slots at the shortest span
    blocks = sum(-(-L // 16) for L in lens) * 8
    span = -(-blocks // 512)
    assert p.max_splits >= -(-(-(-max(lens) // 16)) // span) + 1
    assert fd.plan_splits(d, [8192] * 32, num_cus=256).spans == 0          # equal lengths
    assert fd.plan_splits(d, lens, num_cus=4096).spans == 0                # one round of tiles
    d32 = fd.make_dims(32, 64, 8, 128, 1, 8192, fd.FD_F32)
    assert fd.plan_splits(d32, lens, num_cus=256).spans == 0               # vector kernel
    dq = fd.make_dims(32, 64, 8, 128, 8, 8192, fd.FD_BF16)
    assert fd.plan_splits(dq, lens, num_cus=256).spans == 0                # 64-row chunks: chunk kernel
    assert fd.plan_splits(d, lens, num_splits=4, num_cus=256).spans == 0   # forced count
    # a pair of 2^23 bf16 rows at D = 128 would reach 2^31 bytes in one piece
    big = [1 << 22, 1000, 5000, 300]
    assert fd.plan_splits(fd.make_dims(4, 64, 8, 128, 1, (1 << 23) - 16, fd.FD_BF16), big, num_cus=4).spans > 0
    assert fd.plan_splits(fd.make_dims(4, 64, 8, 128, 1, 1 << 23, fd.FD_BF16), big, num_cus=4).spans == 0


def test_partials_and_combine_reject_bad_arguments(lib):
    d = dims(Lmax=64)
    q, k, v, lens, o, m = FAKE[:6]
    # neither a split count nor a plan
    assert lib.fd_decode_partials(ctypes.byref(d), q, k, v, lens, ctypes.c_float(1.0), 0, None,
                                  o, m, FAKE[6], None) == fd.FD_ERR_INVALID
    assert lib.fd_decode_partials(ctypes.byref(d), q, k, v, lens, ctypes.c_float(1.0), 4, None,
                                  None, m, FAKE[6], None) == fd.FD_ERR_INVALID
    assert lib.fd_combine_splits(1, 32, 1, 128, 0, FAKE[0], FAKE[1], None, fd.FD_BF16, FAKE[2], None,
                                 None) == fd.FD_ERR_INVALID
    assert lib.fd_combine_splits(1, 32, 1, 128, 257, FAKE[0], FAKE[1], None, fd.FD_BF16, FAKE[2], None,
                                 None) == fd.FD_ERR_INVALID
    assert lib.fd_combine_splits(1, 32, 1, 96, 4, FAKE[0], FAKE[1], None, fd.FD_BF16, FAKE[2], None,
                                 None) == fd.FD_ERR_UNSUPPORTED
    assert lib.fd_combine_splits(1, 32, 1, 128, 4, None, FAKE[1], None, fd.FD_BF16, FAKE[2], None,
                                 None) == fd.FD_ERR_INVALID
    assert lib.fd_combine_splits(1, 32, 1, 128, 4, FAKE[0], FAKE[1], None, 5, FAKE[2], None,
                                 None) == fd.FD_ERR_UNSUPPORTED


def test_combine_rejects_misaligned_splits_per_seq(lib):
    odd = ctypes.c_void_p(FAKE[3].value + 2)
    assert lib.fd_combine_splits(1, 32, 1, 128, 4, FAKE[0], FAKE[1], odd, fd.FD_BF16, FAKE[2], None,
                                 None) == fd.FD_ERR_INVALID
    assert "splits_per_seq" in lib.fd_last_error().decode()


def test_tiles_of_2gib_or_more_are_rejected(lib):
    """Tiles are addressed with 32-bit byte offsets: a split rule under which
    one tile of one KV head reaches 2^31 bytes is refused before any launch,
    for every entry point and cache format."""
    L = 1 << 23  # bf16 keys at D = 128: 2^23 * 256 B = 2^31 B
    d = dims(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=L)
    # one tile holding every key (no plan): 2^31 bytes
    assert call_decode(lib, d) == fd.FD_ERR_UNSUPPORTED
    assert "2^31" in lib.fd_last_error().decode()
    # two forced splits: 2^30 bytes each -- passes the check, fails later on
    # the missing workspace
    assert call_decode(lib, d, num_splits=2) == fd.FD_ERR_WORKSPACE
    # a plan whose last tile takes the rest of the keys: 2^23 + 2^20 keys in
    # two slots of 2^20 leave 2^23 keys (2^31 bytes) to the last tile
    d_long = dims(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=L + (1 << 20))
    p = fd.FdPlan(tile_len=1 << 20, max_splits=2)
    assert call_decode(lib, d_long, plan=p) == fd.FD_ERR_UNSUPPORTED
    p = fd.FdPlan(tile_len=1 << 20, max_splits=3)  # last tile 2^23 - 2^20 keys
    assert call_decode(lib, d_long, plan=p) == fd.FD_ERR_WORKSPACE
    # the same plan with balanced spans: a piece may hold a whole pair
    # (2^23 + 2^20 keys) when few workgroups are resident, so it is refused;
    # below 2^23 keys the span plan passes
    p = fd.FdPlan(tile_len=1 << 20, max_splits=3, spans=64)
    assert call_decode(lib, d_long, plan=p) == fd.FD_ERR_UNSUPPORTED
    assert "2^31" in lib.fd_last_error().decode()
    d_short = dims(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=L - 16)
    assert call_decode(lib, d_short, plan=p) == fd.FD_ERR_WORKSPACE
    # one-byte codes hold twice the keys per byte: one tile of 2^23 codes at
    # D = 128 is 2^30 bytes and passes (the misaligned out stops the call
    # before any launch)
    odd_out = ctypes.c_void_p(FAKE[4].value + 8)
    assert lib.fd_decode_attention_fp8(ctypes.byref(d), *FAKE[:3], None, ctypes.c_float(1.0), ctypes.c_float(1.0),
                                       FAKE[3], ctypes.c_float(1.0), 0, None, None, 0, odd_out, None,
                                       None) == fd.FD_ERR_INVALID
    d2 = dims(B=1, Hq=32, Hkv=8, D=128, T=1, Lmax=1 << 24)
    assert lib.fd_decode_attention_fp8(ctypes.byref(d2), *FAKE[:3], None, ctypes.c_float(1.0), ctypes.c_float(1.0),
                                       FAKE[3], ctypes.c_float(1.0), 0, None, None, 0, FAKE[4], None,
                                       None) == fd.FD_ERR_UNSUPPORTED
    # fp32 rows are twice as long
    d3 = dims(B=1, Hq=8, Hkv=8, D=128, T=1, Lmax=1 << 22, dt=fd.FD_F32)
    assert call_decode(lib, d3) == fd.FD_ERR_UNSUPPORTED
    assert lib.fd_decode_partials(ctypes.byref(d3), *FAKE[:4], ctypes.c_float(1.0), 1, None, FAKE[4], FAKE[5],
                                  FAKE[6], None) == fd.FD_ERR_UNSUPPORTED


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """fd_decode_attention_noalloc refuses a call whose partials exceed the
    static scratch before looking it up or launching anything."""
    d = dims(B=64, Hq=64, Hkv=8, D=128, T=1, Lmax=1024)
    assert lib.fd_workspace_bytes(ctypes.byref(d), 256) > fd.FD_NOALLOC_SCRATCH_BYTES
    st = lib.fd_decode_attention_noalloc(ctypes.byref(d), *FAKE[:4], ctypes.c_float(0.1), 256, None, FAKE[4],
                                         FAKE[5], None)
    assert st == fd.FD_ERR_WORKSPACE
    assert "static scratch" in lib.fd_last_error().decode()
    # the usual validation comes first
    st = lib.fd_decode_attention_noalloc(ctypes.byref(d), None, *FAKE[1:4], ctypes.c_float(0.1), 256, None,
                                         FAKE[4], FAKE[5], None)
    assert st == fd.FD_ERR_INVALID


def test_stream_read_rejects_bad_arguments(lib):
    assert lib.fd_stream_read(FAKE[0], 100, 0, 0, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(None, 1024, 0, 0, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(FAKE[0], 1024, -1, 0, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(FAKE[0], 1024, 8, 2, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(FAKE[0], 1024, 8, -1, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(ctypes.c_void_p(FAKE[0].value + 8), 1024, 8, 0, FAKE[1], None) == fd.FD_ERR_INVALID
    assert lib.fd_stream_read(FAKE[0], 1024, 8, 0, None, None) == fd.FD_ERR_INVALID
    # nothing to read: no launch, no pointer touched
    assert lib.fd_stream_read(None, 0, 0, 0, None, None) == fd.FD_OK


def test_empty_batch_is_a_no_op(lib):
    d = dims(B=0)
    # nothing to do: OK without touching any pointer
    assert lib.fd_decode_attention(ctypes.byref(d), None, None, None, None, ctypes.c_float(1.0), 0,
                                   None, None, 0, None, None, None) == fd.FD_OK
    assert lib.fd_combine_splits(0, 4, 1, 64, 2, None, None, None, fd.FD_F32, None, None, None) == fd.FD_OK


def _up(x):
    return math.ceil(x / 256) * 256


def test_workspace_layout_size():
    d = dims(B=2, Hq=8, Hkv=2, D=64, T=3, Lmax=100, dt=fd.FD_F32)
    rows = 2 * 8 * 3
    S = 5
    expect = _up(rows * S * 64 * 4) + 2 * _up(rows * S * 4)
    assert fd.workspace_bytes(d, S) == expect
    assert fd.workspace_bytes(d, 1) == 0
    d = dims(B=3, Hq=32, Hkv=8, D=128, T=1, Lmax=100, dt=fd.FD_BF16)
    rows = 3 * 32
    expect = _up(rows * S * 128 * 4) + 2 * _up(rows * S * 4)
    assert fd.workspace_bytes(d, S) == expect


def call_paged(lib, d, pages, num_splits=0, plan=None, ws=None, ws_bytes=0):
    q, k, v, lens, o, lse = FAKE[:6]
    return lib.fd_decode_attention_paged(ctypes.byref(d), q, k, v,
                                         ctypes.byref(pages) if pages is not None else None, lens,
                                         ctypes.c_float(0.1), num_splits,
                                         ctypes.byref(plan) if plan is not None else None, ws, ws_bytes,
                                         o, lse, None)


def test_paged_rejects_bad_page_descriptions(lib):
    d = dims(Lmax=64)  # 4 pages of 16 keys
    ok = dict(block_table=FAKE[7].value, max_pages_per_seq=4, page_size=16, num_pages=10,
              layout=fd.FD_PAGES_NHD)

    def pages(**kw):
        a = dict(ok)
        a.update(kw)
        return fd.FdKvPages(**a)

    assert call_paged(lib, d, None) == fd.FD_ERR_INVALID
    assert call_paged(lib, d, pages(block_table=None)) == fd.FD_ERR_INVALID
    assert call_paged(lib, d, pages(block_table=0x100002)) == fd.FD_ERR_INVALID
    assert call_paged(lib, d, pages(num_pages=0)) == fd.FD_ERR_INVALID
    assert call_paged(lib, d, pages(max_pages_per_seq=0)) == fd.FD_ERR_INVALID
    assert call_paged(lib, d, pages(max_pages_per_seq=3)) == fd.FD_ERR_INVALID  # 48 != 64
    assert "max_cache_len" in lib.fd_last_error().decode()
    assert call_paged(lib, fd.make_dims(1, 32, 8, 128, 1, 96, fd.FD_BF16),
                      pages(page_size=24, max_pages_per_seq=4)) == fd.FD_ERR_UNSUPPORTED
    assert call_paged(lib, fd.make_dims(1, 32, 8, 128, 1, 32, fd.FD_BF16),
                      pages(page_size=8)) == fd.FD_ERR_UNSUPPORTED
    assert call_paged(lib, d, pages(layout=2)) == fd.FD_ERR_UNSUPPORTED
    # tiles must start at multiples of 16 keys
    assert call_paged(lib, d, pages(), plan=fd.FdPlan(tile_len=40, max_splits=2)) == fd.FD_ERR_INVALID
    # the common checks still apply
    assert call_paged(lib, dims(D=96, Lmax=64), pages()) == fd.FD_ERR_UNSUPPORTED
    assert call_paged(lib, d, pages(), num_splits=4) == fd.FD_ERR_WORKSPACE


def test_paged_empty_batch_is_a_no_op(lib):
    d = dims(B=0, Lmax=64)
    pages = fd.FdKvPages(FAKE[7].value, 4, 16, 10, fd.FD_PAGES_HND)
    assert lib.fd_decode_attention_paged(ctypes.byref(d), None, None, None, ctypes.byref(pages), None,
                                         ctypes.c_float(1.0), 0, None, None, 0, None, None, None) == fd.FD_OK


def test_fp8_rejects_unsupported_calls(lib):
    q, k, v, lens, o, lse = FAKE[:6]

    def call(d, ks=1.0, vs=1.0):
        return lib.fd_decode_attention_fp8(ctypes.byref(d), q, k, v, None, ctypes.c_float(ks), ctypes.c_float(vs),
                                           lens, ctypes.c_float(0.1), 0, None, None, 0, o, lse, None)

    assert call(dims(Lmax=64, dt=fd.FD_F32)) == fd.FD_ERR_UNSUPPORTED        # q must be bf16
    assert "bf16" in lib.fd_last_error().decode()
    assert call(dims(Lmax=64), ks=float("inf")) == fd.FD_ERR_INVALID
    assert call(dims(Lmax=64), vs=float("nan")) == fd.FD_ERR_INVALID
    assert call(dims(D=96, Lmax=64)) == fd.FD_ERR_UNSUPPORTED
    assert lib.fd_decode_partials_fp8(ctypes.byref(dims(Lmax=64)), q, k, v, None, ctypes.c_float(1.0),
                                      ctypes.c_float(1.0), lens, ctypes.c_float(0.1), 0, None, o, FAKE[6],
                                      FAKE[7], None) == fd.FD_ERR_INVALID     # neither splits nor plan
