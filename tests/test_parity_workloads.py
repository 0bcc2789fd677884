"""GPU parity of the one-byte and paged cache paths at the benchmark
workloads' shapes, in the launch configuration the benchmark times (the
planner's plan), every output row against the fp64 oracle at the flat
tolerance (2e-3 on out and lse) with the rel-L2 guard.

Shapes: the 32-sequence variable-length batch (lengths U[512, 8192]; on a
256-CU device the planner cuts it into balanced spans, one per resident
workgroup) and the 4 x 128k batch (16384-key tiles, which give each wave of
the one-byte decode kernel 128 blocks); FP8
E4M3 and INT8 caches (per-tensor scales) and 16-key pages in both layouts.
Page "ChunkedPrefill与FlashDecoding技术解析" §4.2 item 1 asks for exactly this
check: the tiled result against the full one on the same seeded inputs.
"""
import functools

import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import (WORKLOADS, as_oracle_array, fp8_scale_for, int8_scale_for, paginate,
                                            quantize_fp8, quantize_int8, workload_inputs)
from gpu_cases import compare_workload, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

SHAPES = ["varlen_b32", "gqa_128k_b4"]


@functools.lru_cache(maxsize=2)
def _inputs(name):
    return workload_inputs(WORKLOADS[name])


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("name", SHAPES)
def test_one_byte_caches_at_workload(name, fmt):
    w = WORKLOADS[name]
    say(f"[case] {fmt} caches, workload {w.name} (planner tiles, every row)")
    q, k, v, cl = _inputs(name)
    scale_for, quantize, attn, ref_fn = {
        "fp8": (fp8_scale_for, quantize_fp8, fd.decode_attention_fp8, oracle.attention_fp8),
        "int8": (int8_scale_for, quantize_int8, fd.decode_attention_int8, oracle.attention_int8),
    }[fmt]
    ks, vs = scale_for(k), scale_for(v)
    kc, vc = quantize(k, ks), quantize(v, vs)
    plan = fd.plan_for(q, kc, cl)
    say(f"  plan {plan.plan} k_scale {ks:.6g} v_scale {vs:.6g}")
    ref_out, ref_lse = ref_fn(as_oracle_array(q), kc.numpy(), vc.numpy(), cl.numpy(), w.scale, ks, vs)
    kd, vd = kc.cuda(), vc.cuda()
    del kc, vc
    out, lse = attn(q.cuda(), kd, vd, cl.cuda(), ks, vs, scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    compare_workload(f"{fmt} {w.name}", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("name", SHAPES)
def test_paged_16_at_workload(name, layout):
    """16-key pages in a shuffled pool, read in place: every row against the
    oracle, and bit-equal to the contiguous path with the same plan."""
    w = WORKLOADS[name]
    say(f"[case] paged workload {w.name}, 16-key pages, {layout}")
    q, k, v, cl = _inputs(name)
    pc = paginate(k, v, cl, 16, layout, seed=w.seed)
    dims, _ = fd.paged_dims(q, pc.k_pages, pc.block_table, layout)
    plan = fd.plan_splits(dims, cl)
    say(f"  plan {plan.plan}, {pc.k_pages.shape[0]} pages")
    ref_out, ref_lse = oracle.attention_paged(as_oracle_array(q), as_oracle_array(pc.k_pages),
                                              as_oracle_array(pc.v_pages), pc.block_table.numpy(), cl.numpy(),
                                              w.scale, layout)
    qd, cld = q.cuda(), cl.cuda()
    kp, vp, tb = pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda()
    del pc
    out, lse = fd.decode_attention_paged(qd, kp, vp, tb, cld, layout=layout, scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    compare_workload(f"paged16 {layout} {w.name}", out, lse, ref_out, ref_lse)
    del kp, vp
    co, cls = fd.decode_attention(qd, k.cuda(), v.cuda(), cld, scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), co.view(torch.int16)), "paged and contiguous outputs differ"
    assert torch.equal(lse, cls), "paged and contiguous lse differ"
