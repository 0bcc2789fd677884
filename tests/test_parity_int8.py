"""GPU parity of the INT8 cache path (fd_decode_attention_int8,
fd_decode_partials_int8) against the fp64 oracle's definition over
dequantised caches (key = code * k_scale, value = code * v_scale).

Caches are the seeded N(0, 1) draws quantised once, on the host, with a
symmetric per-tensor scale (largest |value| -> 127); both sides read the same
codes.  INT8 has no NaN code, so padding past each sequence's length holds
127, the largest code: read by mistake, it takes over the softmax of every
query row whose elements sum above zero and moves the output far outside the
tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import (WORKLOADS, as_oracle_array, int8_scale_for, make_inputs, paginate,
                                            quantize_int8, workload_inputs)
from gpu_cases import TOL, compare, compare_workload, rel_l2_guard_for, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def int8_inputs(B, Hq, Hkv, D, T, Lmax, seed, lens, q_mul=1.0):
    q, k, v, cl = make_inputs(B, Hq, Hkv, D, T, Lmax, "bf16", seed, cache_lens=lens)
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(torch.bfloat16)
    ks, vs = int8_scale_for(k), int8_scale_for(v)
    kc, vc = quantize_int8(k, ks), quantize_int8(v, vs)
    for b, L in enumerate(cl.tolist()):
        kc[b, :, L:] = 127
        vc[b, :, L:] = 127
    return q, kc, vc, cl, ks, vs


def oracle_int8(q, kc, vc, cl, sc, ks, vs):
    return oracle.attention_int8(as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy(), sc, ks, vs)


def check_int8(name, B, Hq, Hkv, D, T, Lmax, seed, lens, num_splits=0, use_plan=False, page=None, q_mul=1.0):
    say(f"[case] int8 {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} q_len={T} Lmax={Lmax} "
        f"lens={lens if len(lens) <= 8 else str(lens[:8]) + '...'} splits={num_splits} plan={use_plan} page={page}")
    q, kc, vc, cl, ks, vs = int8_inputs(B, Hq, Hkv, D, T, Lmax, seed, lens, q_mul)
    sc = _scale(D)
    ref_out, ref_lse = oracle_int8(q, kc, vc, cl, sc, ks, vs)
    plan = fd.plan_for(q, kc, cl) if use_plan else None
    table, layout = None, "nhd"
    if page is not None:
        P, layout = page
        pc = paginate(kc, vc, cl, P, layout, seed=seed + 7)
        kc, vc, table = pc.k_pages, pc.v_pages, pc.block_table.cuda()
    out, lse = fd.decode_attention_int8(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, block_table=table,
                                        layout=layout, scale=sc, num_splits=num_splits, plan=plan)
    torch.cuda.synchronize()
    return compare(name, out, lse, ref_out, ref_lse, TOL["bf16"])


LENS = [1000, 1, 0, 257, 2048, 16, 17]


@pytest.mark.parametrize("D", [128, 64])
def test_int8_decode(D):
    for S, use_plan in ((0, True), (3, False), (1, False), (64, False)):
        check_int8(f"D={D} S={S}", len(LENS), 32, 8, D, 1, 2048, 4000 + D + S, LENS, num_splits=S,
                   use_plan=use_plan)


def test_int8_gqa_ratios_and_short_chunks():
    for Hq, Hkv, T in [(8, 8, 1), (16, 8, 1), (64, 8, 1), (32, 8, 2), (32, 8, 4), (32, 8, 8), (8, 2, 3)]:
        check_int8(f"Hq={Hq} Hkv={Hkv} q_len={T}", 2, Hq, Hkv, 128, T, 700, 4100 + Hq + T, [700, T + 5],
                   num_splits=3)


def test_int8_paged():
    for P, layout in ((16, "nhd"), (64, "hnd"), (256, "nhd")):
        for S, use_plan in ((0, True), (2, False)):
            check_int8(f"paged {P} {layout} S={S}", len(LENS), 32, 8, 128, 1, 2048, 4200 + P + S, LENS,
                       num_splits=S, use_plan=use_plan, page=(P, layout))


def test_int8_peaked_scores():
    check_int8("q x10", 2, 32, 8, 128, 1, 4096, 4300, [4096, 1500], use_plan=True, q_mul=10.0)


def test_int8_partials_then_combine_equal_whole_call():
    say("[case] int8 partials + combine == fd_decode_attention_int8")
    q, kc, vc, cl, ks, vs = int8_inputs(3, 32, 8, 128, 1, 3000, 4400, [3000, 100, 0])
    qd, kd, vd, cld = q.cuda(), kc.cuda(), vc.cuda(), cl.cuda()
    o_p, m_p, l_p = fd.decode_partials_int8(qd, kd, vd, cld, ks, vs, scale=_scale(128), num_splits=6)
    out, lse = fd.combine(o_p, l_p, out_dtype=torch.bfloat16)
    out2, lse2 = fd.decode_attention_int8(qd, kd, vd, cld, ks, vs, scale=_scale(128), num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    compare("int8 partials+combine", out, lse, *oracle_int8(q, kc, vc, cl, _scale(128), ks, vs), TOL["bf16"])


def test_int8_headline_shape():
    """The 32k GQA decode step over INT8 caches: every row against the oracle."""
    w = WORKLOADS["gqa_32k"]
    say(f"[case] int8 workload {w.name}")
    q, k, v, cl = workload_inputs(w)
    ks, vs = int8_scale_for(k), int8_scale_for(v)
    kc, vc = quantize_int8(k, ks), quantize_int8(v, vs)
    del k, v
    plan = fd.plan_for(q, kc, cl)
    say(f"  plan {plan.plan} k_scale {ks:.6g} v_scale {vs:.6g}")
    ref_out, ref_lse = oracle_int8(q, kc, vc, cl, w.scale, ks, vs)
    out, lse = fd.decode_attention_int8(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, scale=w.scale,
                                        plan=plan)
    torch.cuda.synchronize()
    compare_workload("int8 gqa_32k", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("D", [128, 64])
def test_int8_long_chunks(D):
    """Row groups of more than 32 rows over INT8 caches: the chunk kernel's
    code ring, dequantised a stage ahead."""
    for T, Hq, Hkv, lens in [(33, 1, 1, [40, 33]), (100, 4, 1, [900, 100]), (200, 4, 2, [1500, 150])]:
        for S in (1, 3):
            check_int8(f"chunk q_len={T} Hq={Hq} Hkv={Hkv} D={D} S={S}", len(lens), Hq, Hkv, D, T, max(lens),
                       4500 + T + S, lens, num_splits=S)
    check_int8(f"chunk planned D={D}", 2, 8, 2, D, 96, 2000, 4590, [2000, 96], use_plan=True)
    check_int8(f"chunk paged 16 nhd D={D}", 2, 8, 2, D, 64, 1024, 4592, [1024, 100], num_splits=2,
               page=(16, "nhd"))


def test_int8_prefill_workload():
    """The 512-query prefill chunk over INT8 caches: every row against the oracle."""
    w = WORKLOADS["prefill_chunk_512"]
    say(f"[case] int8 workload {w.name}")
    q, k, v, cl = workload_inputs(w)
    ks, vs = int8_scale_for(k), int8_scale_for(v)
    kc, vc = quantize_int8(k, ks), quantize_int8(v, vs)
    del k, v
    plan = fd.plan_for(q, kc, cl)
    ref_out, ref_lse = oracle_int8(q, kc, vc, cl, w.scale, ks, vs)
    out, lse = fd.decode_attention_int8(q.cuda(), kc.cuda(), vc.cuda(), cl.cuda(), ks, vs, scale=w.scale,
                                        plan=plan)
    torch.cuda.synchronize()
    compare_workload("int8 prefill_chunk_512", out, lse, ref_out, ref_lse, guard=rel_l2_guard_for(4 * 512))
