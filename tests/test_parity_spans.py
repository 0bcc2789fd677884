"""GPU parity of the decode kernel's balanced-span mode (plans with spans > 0)
against the fp64 oracle: every slot's partial against the oracle's split form
over the same key ranges (``oracle.span_ranges``, written from the cut rule),
the empty slots, and whole calls over bf16, FP8, INT8 and paged caches.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import (as_oracle_array, fp8_scale_for, int8_scale_for, paginate, quantize_fp8,
                                            quantize_int8)
from gpu_cases import TOL, compare, compare_workload, inputs, run_oracle, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

SENTINEL = 12345.0


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def _span_plan(spans, slots):
    return fd.FdPlan(tile_len=256, max_splits=slots, spans=spans)


PARTIAL_CASES = [
    # name, B, Hq, Hkv, D, q_len, lens, spans, slots
    ("n_rep 4", 6, 8, 2, 128, 1, [1000, 77, 0, 640, 33, 2000], 7, 4),
    ("D64 n_rep 4", 6, 8, 2, 64, 1, [1000, 77, 0, 640, 33, 2000], 7, 4),
    ("causal 4x3 rows", 5, 8, 2, 128, 3, [900, 3, 0, 257, 1500], 11, 5),
    ("two row blocks (24 rows)", 4, 16, 2, 128, 3, [700, 40, 1300, 16], 9, 4),
    ("one span", 3, 4, 4, 128, 1, [500, 0, 129], 1, 2),
    ("short sequences", 8, 8, 2, 64, 1, [1, 15, 16, 17, 31, 32, 33, 0], 13, 3),
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: c[0])
def test_span_partials_match_oracle_ranges(case):
    name, B, Hq, Hkv, D, T, lens, spans, slots = case
    say(f"[case] span partials {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} q_len={T} spans={spans} slots={slots}")
    Lmax = max(lens)
    q, k, v, cl = inputs(B, Hq, Hkv, D, T, Lmax, "bf16", 4100 + B + D + T, lens, poison=True)
    sc = _scale(D)
    o_p = torch.full((B, Hq, T, slots, D), SENTINEL, dtype=torch.float32, device="cuda")
    o_p, m_p, l_p = fd.decode_partials(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=sc,
                                       plan=_span_plan(spans, slots), o_part=o_p)
    torch.cuda.synchronize()
    lo, hi, per = oracle.span_ranges(cl.numpy(), Hkv, spans, slots, piece_blocks=16)  # the rule's piece cost
    _, _, ro, rm, rl = oracle.attention_ranges(as_oracle_array(q), as_oracle_array(k), as_oracle_array(v),
                                               cl.numpy(), sc, lo, hi)
    say(f"  cut length {per} blocks; slots written: {int(np.isfinite(rl).sum())} finite of {rl.size}")
    gm, gl = m_p.cpu().double().numpy(), l_p.cpu().double().numpy()
    assert np.array_equal(np.isinf(gm), np.isinf(rm)) and np.array_equal(np.isinf(gl), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(gm[fin] - rm[fin]), initial=0.0) <= TOL["bf16"]
    assert np.max(np.abs(gl[fin] - rl[fin]), initial=0.0) <= TOL["bf16"]
    go = o_p.cpu().double().numpy()
    assert np.max(np.abs(go[fin] - ro[fin]), initial=0.0) <= TOL["bf16"]
    assert (go[~fin] == SENTINEL).all(), "an empty slot's o_part entry was written"


WHOLE_CASES = [
    ("ragged", 6, 32, 8, 128, 1, [1000, 77, 0, 640, 33, 2000]),
    ("verify 4 rows", 5, 32, 8, 128, 4, [900, 4, 0, 257, 1500]),
    ("D64 n_rep 8", 4, 16, 2, 64, 1, [2048, 1, 700, 0]),
]


@pytest.mark.parametrize("case", WHOLE_CASES, ids=lambda c: c[0])
def test_span_planned_calls_match_oracle(case):
    """The planner's own span plan (mixed lengths, planned for 4 compute
    units so these small batches outnumber two tiles per unit), whole call,
    bf16 caches."""
    name, B, Hq, Hkv, D, T, lens = case
    say(f"[case] span planned {name}")
    q, k, v, cl = inputs(B, Hq, Hkv, D, T, max(lens), "bf16", 4200 + B + D, lens, poison=True)
    plan = fd.plan_for(q, k, cl, num_cus=4)
    say(f"  plan {plan.plan}")
    assert plan.spans > 0
    ref = run_oracle(q, k, v, cl, _scale(D))
    out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(D), plan=plan)
    torch.cuda.synchronize()
    compare(f"span {name}", out, lse, *ref, TOL["bf16"])


def test_span_count_above_resident_workgroups():
    """A plan asking for more spans than workgroups fit on the device: the
    launch cuts fewer, larger spans (a partition these partial checks cannot
    name in advance), so the whole call is checked."""
    lens = [3000, 2999, 17, 1, 0, 1500]
    say(f"[case] 5000 spans asked, lens={lens}")
    q, k, v, cl = inputs(len(lens), 32, 8, 128, 1, 3000, "bf16", 4250, lens, poison=True)
    plan = _span_plan(5000, 5)
    out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(128), plan=plan)
    torch.cuda.synchronize()
    compare("span 5000 asked", out, lse, *run_oracle(q, k, v, cl, _scale(128)), TOL["bf16"])


def test_span_large_ragged_batch_and_empty_batch():
    """200 short sequences (every workgroup scans the whole batch), then a
    batch whose sequences all have no keys (every slot padded)."""
    rng = np.random.Generator(np.random.PCG64(4260))
    lens = rng.integers(0, 300, size=200).tolist()
    say(f"[case] span 200 sequences, sum {sum(lens)}")
    q, k, v, cl = inputs(200, 8, 2, 64, 1, 300, "bf16", 4261, lens, poison=True)
    plan = _span_plan(64, 4)
    out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(64), plan=plan)
    torch.cuda.synchronize()
    compare("span 200 sequences", out, lse, *run_oracle(q, k, v, cl, _scale(64)), TOL["bf16"])
    say("[case] span batch without keys")
    q, k, v, cl = inputs(3, 8, 2, 64, 1, 64, "bf16", 4262, [0, 0, 0])
    out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(64), plan=_span_plan(16, 3))
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("dt,T", [("f32", 1), ("bf16", 40)])
def test_span_plans_on_tile_kernels(dt, T):
    """A span plan handed to a call that the decode kernel does not serve
    (fp32 caches: the vector kernel; 320 rows per KV head: the chunk kernel)
    runs the plan's tiles."""
    lens = [1000, 77, 0, 640]
    say(f"[case] span plan on the {'vector' if dt == 'f32' else 'chunk'} kernel")
    q, k, v, cl = inputs(4, 16, 2, 128, T, 1000, dt, 4270 + T, lens)
    plan = _span_plan(9, 4)
    out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=_scale(128), plan=plan)
    torch.cuda.synchronize()
    compare(f"span plan, {dt} q_len {T}", out, lse, *run_oracle(q, k, v, cl, _scale(128)), TOL[dt])


@pytest.mark.parametrize("codes", ["fp8", "int8"])
def test_span_one_byte_caches(codes):
    lens = [3000, 100, 0, 1777, 16]
    say(f"[case] span {codes} caches lens={lens}")
    q, k, v, cl = inputs(len(lens), 32, 8, 128, 1, 3000, "bf16", 4300, lens)
    scale_for, quantize = (fp8_scale_for, quantize_fp8) if codes == "fp8" else (int8_scale_for, quantize_int8)
    ks, vs = scale_for(k), scale_for(v)
    kc, vc = quantize(k, ks), quantize(v, vs)
    plan = _span_plan(37, 5)
    attn = fd.decode_attention_fp8 if codes == "fp8" else fd.decode_attention_int8
    out, lse = attn(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, scale=_scale(128), plan=plan)
    torch.cuda.synchronize()
    ref_fn = oracle.attention_fp8 if codes == "fp8" else oracle.attention_int8
    ref = ref_fn(as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy(), _scale(128), ks, vs)
    compare(f"span {codes}", out, lse, *ref, TOL["bf16"])


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
def test_span_paged_equals_contiguous(layout):
    """Span partials over pages: bit-equal to the contiguous caches' span
    partials (same keys in the same order), whole call against the oracle."""
    lens = [1000, 77, 0, 640]
    say(f"[case] span paged {layout}")
    q, k, v, cl = inputs(4, 8, 2, 128, 1, 1024, "bf16", 4400, lens)
    pc = paginate(k, v, cl, 32, layout, seed=4401)
    plan = _span_plan(9, 4)
    sc = _scale(128)
    o_p, m_p, l_p = fd.decode_partials_paged(q.cuda(), pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda(),
                                             cl.cuda(), layout=layout, scale=sc, plan=plan)
    co, cm, cl_ = fd.decode_partials(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=sc, plan=plan)
    out, lse = fd.decode_attention_paged(q.cuda(), pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda(),
                                         cl.cuda(), layout=layout, scale=sc, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(m_p, cm) and torch.equal(l_p, cl_)
    fin = torch.isfinite(l_p)
    assert torch.equal(o_p[fin], co[fin])
    compare(f"span paged {layout}", out, lse, *run_oracle(q, k, v, cl, sc), TOL["bf16"])


COMBO_CASES = [
    # codes, page (size, layout) or None, q_len, D, Hq, Hkv
    ("fp8", (16, "nhd"), 3, 64, 16, 4),
    ("int8", (32, "hnd"), 1, 128, 32, 8),
    (None, (16, "hnd"), 2, 64, 16, 2),
    ("fp8", None, 4, 128, 64, 8),
]


@pytest.mark.parametrize("case", COMBO_CASES, ids=lambda c: f"{c[0]}-{c[1]}-q{c[2]}-D{c[3]}")
def test_span_combinations(case):
    """Spans with one-byte codes, pages, causal chunks, both head dims and
    up to 32 rows per KV head, whole calls against the oracle."""
    codes, page, T, D, Hq, Hkv = case
    lens = [1500, 3, 0, 700, 129, 2048]
    lens = [max(L, T) if L else 0 for L in lens]
    say(f"[case] span combination {case}")
    q, k, v, cl = inputs(len(lens), Hq, Hkv, D, T, 2048, "bf16", 4300 + D + T, lens)
    sc = _scale(D)
    plan = _span_plan(23, 5)
    if codes:
        scale_for, quantize = (fp8_scale_for, quantize_fp8) if codes == "fp8" else (int8_scale_for, quantize_int8)
        ks, vs = scale_for(k), scale_for(v)
        kc, vc = quantize(k, ks), quantize(v, vs)
        ref_fn = oracle.attention_fp8 if codes == "fp8" else oracle.attention_int8
        ref = ref_fn(as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy(), sc, ks, vs)
        table, layout = None, "nhd"
        if page is not None:
            pc = paginate(kc, vc, cl, page[0], page[1], seed=4390)
            kc, vc, table, layout = pc.k_pages, pc.v_pages, pc.block_table.cuda(), page[1]
        attn = fd.decode_attention_fp8 if codes == "fp8" else fd.decode_attention_int8
        out, lse = attn(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, block_table=table, layout=layout,
                        scale=sc, plan=plan)
    else:
        ref = run_oracle(q, k, v, cl, sc)
        pc = paginate(k, v, cl, page[0], page[1], seed=4391)
        out, lse = fd.decode_attention_paged(q.cuda(), pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda(),
                                             cl.cuda(), layout=page[1], scale=sc, plan=plan)
    torch.cuda.synchronize()
    compare(f"span {case}", out, lse, *ref, TOL["bf16"])


@pytest.mark.parametrize("codes", ["bf16", "fp8"])
def test_span_plan_forced_on_the_32k_layer(codes):
    """Spans forced on the equal-length 32k layer (B1, Hq32, Hkv8, D128, 32768
    keys), as ``bench.py --spans 512`` times it (512 spans, 64 slots): every
    output row against the fp64 oracle at the flat workload tolerance."""
    from decode_attention_14_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["gqa_32k"]
    say(f"[case] {codes} caches, workload {w.name}, 512 forced spans over 64 slots")
    q, k, v, cl = workload_inputs(w)
    plan = fd.FdPlan(tile_len=1024, max_splits=64, spans=512)
    if codes == "fp8":
        ks, vs = fp8_scale_for(k), fp8_scale_for(v)
        kc, vc = quantize_fp8(k, ks), quantize_fp8(v, vs)
        ref = oracle.attention_fp8(as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy(), w.scale, ks, vs)
        out, lse = fd.decode_attention_fp8(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, scale=w.scale, plan=plan)
    else:
        ref = run_oracle(q, k, v, cl, w.scale)
        out, lse = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    compare_workload(f"{codes} {w.name} 512 spans", out, lse, *ref)
