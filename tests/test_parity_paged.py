"""GPU parity of the paged-cache path (fd_decode_attention_paged) against the
fp64 oracle, which gathers the pages into a contiguous cache by the block
table's definition and applies the plain attention definition.

Every case builds its page pool with ``inputs.paginate``: shuffled page ids,
NaN in the rows of a page past the sequence's length and in spare pages, so a
kernel that reads outside the visible keys shows up as NaN.  With the same
tiles the paged and the contiguous paths do the same arithmetic in the same
order, so where the tiles agree (planner splits, one split) their outputs
must also agree bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import WORKLOADS, as_oracle_array, paginate, workload_inputs
from gpu_cases import TOL, compare, compare_workload, inputs, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def run_paged(q, pc, cl, scale, num_splits=0, plan=None):
    out, lse = fd.decode_attention_paged(q.cuda(), pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda(),
                                         cl.cuda(), layout=pc.layout, scale=scale, num_splits=num_splits,
                                         plan=plan)
    torch.cuda.synchronize()
    return out, lse


def oracle_paged(q, pc, cl, scale):
    return oracle.attention_paged(as_oracle_array(q), as_oracle_array(pc.k_pages), as_oracle_array(pc.v_pages),
                                  pc.block_table.numpy(), cl.numpy(), scale, pc.layout)


def check_paged(name, B, Hq, Hkv, D, T, Lmax, dt, seed, lens, page_size, layout, num_splits=0, use_plan=False,
                q_mul=1.0):
    say(f"[case] paged {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} q_len={T} Lmax={Lmax} {dt} page={page_size} "
        f"{layout} lens={lens if len(lens) <= 8 else str(lens[:8]) + '...'} splits={num_splits} plan={use_plan}")
    q, k, v, cl = inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, lens, q_mul)
    pc = paginate(k, v, cl, page_size, layout, seed=seed + 1)
    sc = _scale(D)
    plan = None
    if use_plan:
        dims, _ = fd.paged_dims(q, pc.k_pages, pc.block_table, layout)
        plan = fd.plan_splits(dims, cl)
    ref_out, ref_lse = oracle_paged(q, pc, cl, sc)
    out, lse = run_paged(q, pc, cl, sc, num_splits, plan)
    compare(name, out, lse, ref_out, ref_lse, TOL[dt])
    if num_splits in (0, 1):
        # Same tiles as the contiguous path: same bits.
        co, cl_ = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=sc, num_splits=num_splits,
                                      plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(co)), f"{name}: paged and contiguous outputs differ"
        assert torch.equal(lse, cl_), f"{name}: paged and contiguous lse differ"


LENS = [1000, 1, 0, 257, 2048, 16, 17]


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_paged_decode_bf16(layout, page_size):
    for S, use_plan in ((0, True), (3, False), (1, False)):
        check_paged(f"bf16 S={S}", len(LENS), 32, 8, 128, 1, 2048, "bf16", 2000 + page_size, LENS, page_size,
                    layout, num_splits=S, use_plan=use_plan)
    check_paged("bf16 D=64", 3, 8, 2, 64, 1, 512, "bf16", 2100 + page_size, [512, 100, 33], page_size, layout,
                use_plan=True)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_decode_f32(layout, D):
    for page_size in (16, 32):
        for S, use_plan in ((0, True), (4, False)):
            check_paged(f"f32 D={D} S={S}", 4, 8, 2, D, 1, 1024, "f32", 2200 + D + page_size, [1024, 3, 500, 0],
                        page_size, layout, num_splits=S, use_plan=use_plan)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
def test_paged_chunks(layout):
    # Short chunks (row groups up to 32 rows) and long ones (chunk tiles).
    for T, Hq, Hkv, dt in [(3, 8, 2, "bf16"), (8, 8, 2, "bf16"), (3, 8, 2, "f32"), (100, 8, 2, "bf16"),
                           (200, 4, 1, "bf16")]:
        for S, use_plan in ((0, True), (2, False)):
            check_paged(f"chunk q_len={T} {dt} S={S}", 2, Hq, Hkv, 128, T, 1024, dt, 2300 + T, [1024, T + 40], 32,
                        layout, num_splits=S, use_plan=use_plan)
    check_paged("chunk D=64 q x10", 1, 4, 1, 64, 80, 512, "bf16", 2390, [500], 16, layout, num_splits=2,
                q_mul=10.0)


def test_paged_headline_shape():
    """The 32k GQA decode step, paged in 16-key pages (NHD): every row against
    the oracle, and bit-equal to the contiguous path with the same plan."""
    w = WORKLOADS["gqa_32k"]
    say(f"[case] paged workload {w.name}, 16-key pages, nhd")
    q, k, v, cl = workload_inputs(w)
    pc = paginate(k, v, cl, 16, "nhd", seed=w.seed)
    dims, _ = fd.paged_dims(q, pc.k_pages, pc.block_table, "nhd")
    plan = fd.plan_splits(dims, cl)
    say(f"  plan {plan.plan}")
    ref_out, ref_lse = oracle_paged(q, pc, cl, w.scale)
    out, lse = run_paged(q, pc, cl, w.scale, plan=plan)
    compare_workload("paged gqa_32k", out, lse, ref_out, ref_lse)
    co, cls = fd.decode_attention(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(co))
    assert torch.equal(lse, cls)


@pytest.mark.parametrize("layout", ["nhd", "hnd"])
def test_paged_partials(layout):
    """The first pass alone over pages: every tile's partials against the
    oracle's split form, and bit-equal to the contiguous first pass."""
    say(f"[case] paged partials {layout}")
    lens = [1000, 77, 0, 640]
    q, k, v, cl = inputs(4, 8, 2, 128, 1, 1024, "bf16", 2500, lens)
    pc = paginate(k, v, cl, 32, layout, seed=2501)
    plan = fd.FdPlan(tile_len=256, max_splits=4)
    sc = _scale(128)
    o_p, m_p, l_p = fd.decode_partials_paged(q.cuda(), pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda(),
                                             cl.cuda(), layout=layout, scale=sc, plan=plan)
    co, cm, cl_ = fd.decode_partials(q.cuda(), k.cuda(), v.cuda(), cl.cuda(), scale=sc, plan=plan)
    torch.cuda.synchronize()
    _, _, ro, rm, rl = oracle.attention_split(as_oracle_array(q), as_oracle_array(k), as_oracle_array(v),
                                              cl.numpy(), sc, tile_len=256, slots=4)
    gm, gl = m_p.cpu().double().numpy(), l_p.cpu().double().numpy()
    assert np.array_equal(np.isinf(gl), np.isinf(rl)) and np.array_equal(np.isinf(gm), np.isinf(rm))
    fin = np.isfinite(rl)
    assert np.max(np.abs(gm[fin] - rm[fin])) <= TOL["bf16"]
    assert np.max(np.abs(gl[fin] - rl[fin])) <= TOL["bf16"]
    assert np.max(np.abs(o_p.cpu().double().numpy()[fin] - ro[fin])) <= TOL["bf16"]
    assert torch.equal(m_p, cm) and torch.equal(l_p, cl_)
    fin_t = torch.from_numpy(fin).cuda()
    assert torch.equal(o_p[fin_t], co[fin_t])
