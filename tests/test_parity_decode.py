"""GPU parity of the HIP split-KV path against the fp64 oracle, through the C ABI.

Workload cases use the seeded shapes of the benchmark workloads in the launch
configuration the benchmark times (planner-chosen splits); the edge cases
sweep lengths around tile and step boundaries, forced split counts, GQA
ratios, head dims, dtypes, chunk lengths, empty sequences and poisoned
padding.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import WORKLOADS, as_oracle_array, workload_inputs
from gpu_cases import (TOL, check_case, compare, compare_workload, inputs, rel_l2_guard_for, run_gpu, run_oracle,
                       say)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


# ---------------------------------------------------------------------------
# Benchmark workloads


def test_workload_mha_tiny_1k():
    w = WORKLOADS["mha_tiny_1k"]
    say(f"[case] workload {w.name}")
    q, k, v, cl = workload_inputs(w)
    ref = run_oracle(q, k, v, cl, w.scale)
    out, lse = run_gpu(q, k, v, cl, w.scale, num_splits=w.num_splits)
    compare_workload(w.name, out, lse, *ref)
    plan = fd.plan_for(q, k, cl)
    out, lse = run_gpu(q, k, v, cl, w.scale, plan=plan)
    compare_workload(w.name + " planned", out, lse, *ref)


@pytest.mark.parametrize("name", ["gqa_32k", "varlen_b32", "gqa_128k_b4", "verify_q4_32k", "prefill_chunk_512"])
def test_workload_full_oracle(name):
    """Every output row of the workload, in the launch configuration the
    benchmark times (planner splits), against the fp64 oracle at the flat
    tolerance; then one tile per sequence (no merge pass)."""
    w = WORKLOADS[name]
    say(f"[case] workload {w.name} (planner splits, whole output against the oracle)")
    q, k, v, cl = workload_inputs(w)
    plan = fd.plan_for(q, k, cl)
    say(f"  plan {plan.plan}")
    ref_out, ref_lse = run_oracle(q, k, v, cl, w.scale)
    out, lse = run_gpu(q, k, v, cl, w.scale, plan=plan)
    guard = rel_l2_guard_for(w.num_q_heads // w.num_kv_heads * w.q_len)
    compare_workload(w.name, out, lse, ref_out, ref_lse, guard)
    del out, lse
    if name != "gqa_128k_b4":  # one 128k-key tile per KV head: covered by the forced-split cases below
        out1, lse1 = run_gpu(q, k, v, cl, w.scale)
        compare_workload(w.name + " one split", out1, lse1, ref_out, ref_lse, guard)


def test_workload_gqa_128k_b4_forced_splits():
    """4 x 128k at forced split counts: 8 tiles of 16384 keys (the planner's
    tile here) and 256 tiles of 512 keys (the slot cap)."""
    w = WORKLOADS["gqa_128k_b4"]
    q, k, v, cl = workload_inputs(w)
    ref_out, ref_lse = run_oracle(q, k, v, cl, w.scale)
    for S in (8, 256):
        say(f"[case] workload {w.name}, {S} forced splits")
        out, lse = run_gpu(q, k, v, cl, w.scale, num_splits=S)
        compare_workload(f"{w.name} S={S}", out, lse, ref_out, ref_lse)


# ---------------------------------------------------------------------------
# Edge cases


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_edge_lengths(dt, D):
    lens_list = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1000]
    for i, L in enumerate(lens_list):
        for S in (1, 3, 7):
            check_case(f"len{L}-S{S}", 1, 8, 2, D, 1, L + 5, dt, 100 + i, [L], num_splits=S)
    check_case("batch of edge lengths planned", len(lens_list), 8, 2, D, 1, 1024, dt, 99,
               lens_list, use_plan=True)


def test_forced_split_counts():
    for S in (1, 2, 3, 4, 7, 64, 256):
        check_case(f"forced S={S}", 2, 16, 4, 128, 1, 2000, "bf16", 200 + S, [777, 2000], num_splits=S)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gqa_ratios(dt):
    for Hq, Hkv in [(4, 4), (8, 4), (6, 2), (8, 2), (10, 2), (16, 2), (32, 2), (16, 1)]:
        for D in (64, 128):
            check_case(f"Hq={Hq} Hkv={Hkv} D={D}", 2, Hq, Hkv, D, 1, 600, dt, 300 + Hq + D,
                       [600, 333], num_splits=3)


def test_varlen_with_empty_and_tiny_sequences():
    lens = [0, 1, 3, 300, 1025, 17, 0, 2048]
    check_case("varlen planned", 8, 16, 4, 128, 1, 2048, "bf16", 400, lens, use_plan=True)
    check_case("varlen forced 5", 8, 16, 4, 128, 1, 2048, "bf16", 401, lens, num_splits=5)
    check_case("varlen one split", 8, 16, 4, 128, 1, 2048, "bf16", 402, lens)
    check_case("all empty", 3, 8, 8, 64, 1, 16, "f32", 403, [0, 0, 0], num_splits=2)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chunk_lengths(dt):
    for T, n_rep in [(2, 1), (3, 1), (5, 1), (2, 4), (3, 4), (17, 1), (17, 4), (64, 4)]:
        check_case(f"q_len={T} n_rep={n_rep}", 2, 2 * n_rep, 2, 128, T, 700, dt, 500 + T * 10 + n_rep,
                   [700, 130], num_splits=3)
    # chunk longer than part of the cache: early rows see nothing
    check_case("q_len > L", 1, 4, 1, 64, 6, 16, dt, 590, [4], num_splits=2)


@pytest.mark.parametrize("D", [128, 64])
def test_long_chunks(D):
    """Row groups of more than 32 rows: the chunk tiles of the matrix-core path."""
    for T, Hq, Hkv, lens in [(33, 1, 1, [40, 33]), (100, 4, 1, [900, 100]), (128, 8, 2, [128, 700]),
                             (200, 4, 2, [1500, 150]), (37, 8, 1, [37, 1000]), (64, 16, 2, [64, 64])]:
        for S in (1, 3):
            check_case(f"chunk q_len={T} Hq={Hq} Hkv={Hkv} D={D} S={S}", len(lens), Hq, Hkv, D, T,
                       max(lens), "bf16", 1400 + T + S, lens, num_splits=S)
    check_case(f"chunk planned D={D}", 2, 8, 2, D, 96, 2000, "bf16", 1490, [2000, 96], use_plan=True)
    check_case(f"chunk q x10 D={D}", 1, 4, 1, D, 80, 900, "bf16", 1491, [900], q_mul=10.0, num_splits=2)
    check_case(f"chunk poison D={D}", 2, 4, 2, D, 48, 400, "bf16", 1492, [300, 60], num_splits=2,
               poison=True)


def test_poisoned_padding():
    for dt in ("bf16", "f32"):
        check_case(f"poison {dt}", 3, 8, 2, 128, 1, 520, dt, 600, [5, 257, 300], num_splits=4,
                   poison=True)
        check_case(f"poison chunk {dt}", 2, 8, 2, 64, 3, 300, dt, 601, [5, 129], num_splits=2,
                   poison=True)


def test_tile_ends_and_plans_from_other_lengths():
    """Tiles whose end is not a multiple of the tile length, and plans made
    from host lengths other than those the device holds (tiles that come out
    empty, a last tile that runs past the plan's tile length).  Padding past
    each length is poisoned (NaN keys, Inf values), so any row read past a
    sequence's end would show."""
    for D in (128, 64):
        # equal lengths below capacity: the last tile is shorter than the others
        check_case(f"short last tile D={D}", 2, 32, 8, D, 1, 3000, "bf16", 1610,
                   [2500, 2500], use_plan=True, poison=True)
    # plans made from other host lengths than the device holds
    for name, host, dev in (("device shorter", [3000, 3000], [2500, 1234]),
                            ("device longer", [1000, 1000], [3000, 2000])):
        say(f"[case] plan from other lengths, {name}: plan lens {host}, device lens {dev}")
        q, k, v, cl = inputs(2, 32, 8, 128, 1, 3000, "bf16", 1611, dev, poison=True)
        plan = fd.plan_for(q, k, torch.tensor(host, dtype=torch.int32))
        ref = run_oracle(q, k, v, cl, _scale(128))
        out, lse = run_gpu(q, k, v, cl, _scale(128), plan=plan)
        compare(f"plan from other lengths, {name}", out, lse, *ref, TOL["bf16"])


@pytest.mark.parametrize("q_len,rows_kernel", [(48, "chunk"), (4, "decode")])
def test_chunk_rows_equal_decode_at_their_lengths(q_len, rows_kernel):
    """Row t of a causal chunk over a cache of L keys is the decode step of
    the same query row over the first L - q_len + t + 1 keys (page
    "ChunkedPrefill与FlashDecoding技术解析" §2.1: a chunk token sees itself
    and earlier positions).  GPU against GPU: a 48-token chunk (192 rows per
    KV head, the matrix-core chunk kernel) or a 4-token one (16 rows, the
    decode kernel's causal path), and single-row decode calls."""
    B, Hq, Hkv, D, L = 2, 16, 4, 128, 1500
    say(f"[case] chunk rows vs decode: q_len={q_len} ({rows_kernel} kernel)")
    q, k, v, cl = inputs(B, Hq, Hkv, D, q_len, L, "bf16", 1700 + q_len, [L, L - 333])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = fd.decode_attention(qd, kd, vd, cl.cuda(), scale=_scale(128),
                                   plan=fd.plan_for(q, k, cl))
    for t in sorted({0, 1, q_len // 2, q_len - 1}):
        lens = torch.tensor([int(x) - q_len + t + 1 for x in cl], dtype=torch.int32)
        q1 = qd[:, :, t:t + 1].contiguous()
        o1, l1 = fd.decode_attention(q1, kd, vd, lens.cuda(), scale=_scale(128),
                                     plan=fd.plan_for(q1.cpu(), k, lens))
        torch.cuda.synchronize()
        d_out = float((out[:, :, t].float() - o1[:, :, 0].float()).abs().max())
        d_lse = float((lse[:, :, t] - l1[:, :, 0]).abs().max())
        assert d_out <= TOL["bf16"] and d_lse <= TOL["bf16"], (t, d_out, d_lse)


def test_peaked_scores():
    check_case("q x10", 2, 32, 8, 128, 1, 4096, "bf16", 700, [4096, 1500], q_mul=10.0, use_plan=True)
    check_case("q x10 f32", 1, 8, 8, 64, 1, 1024, "f32", 701, [1024], q_mul=10.0, num_splits=4)


def test_lengths_above_capacity_are_clamped():
    say("[case] device cache_lens above max_cache_len")
    q, k, v, cl = inputs(2, 8, 2, 64, 1, 100, "f32", 800, [100, 40])
    ref = run_oracle(q, k, v, cl, 0.125)
    big = torch.tensor([1000, 40], dtype=torch.int32)
    out, lse = run_gpu(q, k, v, big, 0.125, num_splits=3)
    compare("clamped lengths", out, lse, *ref, TOL["f32"])


def test_deterministic_bits():
    say("[case] determinism")
    q, k, v, cl = inputs(2, 32, 8, 128, 1, 3000, "bf16", 900, [3000, 1234])
    plan = fd.plan_for(q, k, cl)
    o1, l1 = run_gpu(q, k, v, cl, _scale(128), plan=plan)
    o2, l2 = run_gpu(q, k, v, cl, _scale(128), plan=plan)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_split_count_invariance_on_gpu():
    say("[case] split invariance")
    q, k, v, cl = inputs(1, 32, 8, 128, 1, 4096, "bf16", 901, [4096])
    outs = [run_gpu(q, k, v, cl, _scale(128), num_splits=S)[0].float() for S in (1, 2, 5, 16, 64)]
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) <= 2e-3


# ---------------------------------------------------------------------------
# The two passes separately


@pytest.mark.parametrize("dt,T", [("bf16", 1), ("f32", 1), ("bf16", 3), ("bf16", 40)])
def test_partials_match_oracle_tiles(dt, T):
    say(f"[case] partials {dt} q_len={T}")
    lens = [1000, 77, 0]
    q, k, v, cl = inputs(3, 8, 2, 128, T, 1000, dt, 1000 + T, lens)
    S = 6
    # Slots with no visible key must leave their o_part entries alone.
    sentinel = 12345.0
    o_p = torch.full((3, 8, T, S, 128), sentinel, dtype=torch.float32, device="cuda")
    o_p, m_p, l_p = fd.decode_partials(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(128),
                                       num_splits=S, o_part=o_p)
    torch.cuda.synchronize()
    _, _, ro, rm, rl = oracle.attention_split(as_oracle_array(q), as_oracle_array(k),
                                              as_oracle_array(v), cl.numpy(), _scale(128),
                                              num_splits=S, slots=S)
    say(f"  slots written: {int(np.isfinite(rl).sum())} finite of {rl.size}")
    gm, gl = m_p.cpu().double().numpy(), l_p.cpu().double().numpy()
    assert np.array_equal(np.isinf(gm), np.isinf(rm)) and np.array_equal(np.isinf(gl), np.isinf(rl))
    fin = np.isfinite(rl)
    tol = TOL[dt]
    assert np.max(np.abs(gm[fin] - rm[fin])) <= tol
    assert np.max(np.abs(gl[fin] - rl[fin])) <= tol
    go = o_p.cpu().double().numpy()
    assert np.max(np.abs(go[fin] - ro[fin])) <= tol
    assert (go[~fin] == sentinel).all(), "an empty slot's o_part entry was written"


def test_combine_matches_oracle_merge():
    say("[case] standalone combine")
    rng = np.random.Generator(np.random.PCG64(1100))
    for D, S, (B, H, T) in [(128, 1, (2, 4, 3)), (128, 2, (3, 8, 37)), (64, 3, (3, 8, 37)), (128, 4, (2, 4, 3)),
                            (64, 4, (1, 5, 41)), (128, 7, (2, 4, 3)), (64, 33, (2, 4, 3)), (128, 256, (2, 4, 3))]:
        o = rng.standard_normal((B, H, T, S, D)).astype(np.float32)
        lp = (rng.standard_normal((B, H, T, S)) * 3).astype(np.float32)
        empty = rng.random((B, H, T, S)) < 0.3
        empty[0, 0, 0, :] = True                      # a row with no finite slot
        lp[empty] = -np.inf
        o[empty] = np.nan                             # empty slots may hold anything
        ro, rl = oracle.merge_lse(o.astype(np.float64), lp.astype(np.float64))
        for out_dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-3)):
            go, gl = fd.combine(torch.from_numpy(o).cuda(), torch.from_numpy(lp).cuda(),
                                out_dtype=out_dtype)
            torch.cuda.synchronize()
            compare(f"combine D={D} S={S} rows={B * H * T} {out_dtype}", go, gl, ro, rl, tol)


def test_combine_ragged_splits_per_seq():
    """fd_combine_splits with per-sequence slot counts: sequence b merges only
    its first S_b slots (page "FlashDecoding算法原理与多GPU并行解码实战",
    multi-GPU step 3, where each device may hold a different number of
    partials).  The slots past S_b hold garbage (NaN outputs, large finite
    lse), so reading any of them would show.  Expected: the oracle's merge of
    slots 0 .. S_b - 1; S_b <= 0 gives out = 0, lse = -inf; S_b above the slot
    count is clamped to it."""
    say("[case] standalone combine, ragged splits_per_seq")
    rng = np.random.Generator(np.random.PCG64(1150))
    for D, S, H, T in [(128, 3, 4, 2), (64, 4, 3, 5), (128, 7, 4, 3), (64, 33, 2, 3), (128, 256, 2, 1)]:
        counts = [S, 0, 1, max(1, S // 2), S + 5, -3, S - 1]
        B = len(counts)
        o = rng.standard_normal((B, H, T, S, D)).astype(np.float32)
        lp = (rng.standard_normal((B, H, T, S)) * 3).astype(np.float32)
        lp[rng.random((B, H, T, S)) < 0.2] = -np.inf  # empty slots among the used ones
        ref_o = np.zeros((B, H, T, D))
        ref_l = np.full((B, H, T), -np.inf)
        for b, n in enumerate(counts):
            n = min(max(n, 0), S)
            if n > 0:
                ref_o[b], ref_l[b] = oracle.merge_lse(o[b, :, :, :n].astype(np.float64),
                                                      lp[b, :, :, :n].astype(np.float64))
            o[b, :, :, n:] = np.nan   # slots past the count: garbage
            lp[b, :, :, n:] = 50.0
        spl = torch.tensor(counts, dtype=torch.int32).cuda()
        for out_dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-3)):
            go, gl = fd.combine(torch.from_numpy(o).cuda(), torch.from_numpy(lp).cuda(), out_dtype=out_dtype,
                                splits=spl)
            torch.cuda.synchronize()
            compare(f"ragged combine D={D} S={S} {out_dtype}", go, gl, ref_o, ref_l, tol)


# ---------------------------------------------------------------------------
# Workspace reuse and graph replays


def test_workspace_reuse_with_garbage_and_changing_shapes():
    say("[case] one garbage-filled workspace reused across shapes and split counts")
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    cases = [
        (2, 32, 8, 128, 1, 3000, "bf16", [3000, 1234], 7),
        (1, 32, 8, 128, 1, 5000, "bf16", [5000], 40),
        (4, 16, 2, 64, 1, 900, "bf16", [900, 1, 0, 450], 5),
        (2, 8, 2, 128, 1, 700, "f32", [700, 333], 6),
        (2, 8, 2, 128, 40, 900, "bf16", [900, 100], 3),
        (2, 32, 8, 128, 1, 3000, "bf16", [3000, 1234], 9),
    ]
    for i, (B, Hq, Hkv, D, T, Lmax, dt, lens, S) in enumerate(cases):
        q, k, v, cl = inputs(B, Hq, Hkv, D, T, Lmax, dt, 1200 + i, lens)
        sc = _scale(D)
        ref = run_oracle(q, k, v, cl, sc)
        for rep in range(2):
            out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=sc,
                                           num_splits=S, workspace=ws)
            torch.cuda.synchronize()
            compare(f"reuse case {i} rep {rep}", out, lse, *ref, TOL[dt])


def test_graph_replays_match_eager():
    say("[case] graph replays of the split-KV step")
    q, k, v, cl = inputs(1, 32, 8, 128, 1, 8192, "bf16", 1300, [8192])
    sc = _scale(128)
    qd, kd, vd, cld = q.cuda(), k.cuda(), v.cuda(), cl.cuda()
    plan = fd.plan_for(q, k, cl)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    ws = fd.new_workspace(fd.workspace_bytes(fd.dims_of(qd, kd), plan.max_splits), "cuda")
    fd.decode_attention(qd, kd, vd, cld, scale=sc, plan=plan, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.decode_attention(qd, kd, vd, cld, scale=sc, plan=plan, out=out, lse=lse, workspace=ws)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {rep}: out differs"
        assert torch.equal(lse, eager_lse), f"replay {rep}: lse differs"
        # eager work on the same workspace between replays
        fd.decode_attention(qd, kd, vd, cld, scale=sc, num_splits=5, workspace=ws)
        torch.cuda.synchronize()
    compare("graph replay", out, lse, *run_oracle(q, k, v, cl, sc), TOL["bf16"])


def test_vector_kernel_ablation_switch_in_subprocess():
    """FD_DECODE_KERNEL=vector (read once per process) runs bf16 caches on the
    vector-ALU kernel; FD_TRACE=1 names the kernel.  Parity in a child process."""
    import os
    import subprocess
    import sys
    say("[case] bf16 through the vector kernel (child process)")
    code = (
        "import sys; sys.path.insert(0, 'tests'); sys.path.insert(0, '.')\n"
        "from gpu_cases import check_case\n"
        "check_case('vector bf16 S=3', 2, 32, 8, 128, 1, 3000, 'bf16', 1500, [3000, 777], num_splits=3)\n"
        "check_case('vector bf16 planned', 3, 8, 2, 64, 1, 1000, 'bf16', 1501, [1000, 1, 0], use_plan=True)\n"
        "check_case('vector bf16 chunk', 2, 8, 2, 128, 5, 600, 'bf16', 1502, [600, 20], num_splits=2)\n"
        "print('child ok')\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, FD_DECODE_KERNEL="vector", FD_TRACE="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "child ok" in r.stdout
    assert "fd_partial_kernel (vector)" in r.stderr and "fd_mfma" not in r.stderr


def test_lse_null_through_the_abi():
    """lse may be NULL: the C call with a null lse pointer writes the same out
    bits as with one, for direct single-tile calls (decode and chunk kernels,
    vector kernel) and for split calls that end in the merge."""
    lib = fd.load_library()
    for name, (B, Hq, Hkv, D, T, L, dt), S in [("decode bf16", (2, 32, 8, 128, 1, 900, "bf16"), 1),
                                               ("decode bf16 split", (2, 32, 8, 128, 1, 900, "bf16"), 4),
                                               ("chunk bf16", (1, 8, 2, 128, 40, 500, "bf16"), 1),
                                               ("chunk bf16 split", (1, 8, 2, 128, 40, 500, "bf16"), 3),
                                               ("vector f32 split", (2, 8, 2, 64, 1, 700, "f32"), 3)]:
        say(f"[case] lse NULL: {name}")
        q, k, v, cl = inputs(B, Hq, Hkv, D, T, L, dt, 1400 + S + T, [L, L // 2 + 1][:B])
        qd, kd, vd, cld = q.cuda(), k.cuda(), v.cuda(), cl.cuda()
        sc = _scale(D)
        ref_out, ref_lse = fd.decode_attention(qd, kd, vd, cld, scale=sc, num_splits=S)
        dims = fd.dims_of(qd, kd)
        ws = fd.new_workspace(max(fd.workspace_bytes(dims, S), 256), "cuda")
        out = torch.full_like(qd, float("nan"))
        st = lib.fd_decode_attention(ctypes.byref(dims), fd._ptr(qd), fd._ptr(kd), fd._ptr(vd), fd._ptr(cld),
                                     ctypes.c_float(sc), S, None, fd._ptr(ws), ws.numel(), fd._ptr(out), None,
                                     fd._stream(qd.device))
        torch.cuda.synchronize()
        assert st == fd.FD_OK, lib.fd_last_error().decode()
        bits = torch.int16 if dt == "bf16" else torch.int32
        assert torch.equal(out.view(bits), ref_out.view(bits)), f"{name}: out differs with lse = NULL"
        compare(f"lse NULL {name}", out, ref_lse, *run_oracle(q, k, v, cl, sc), TOL[dt])
