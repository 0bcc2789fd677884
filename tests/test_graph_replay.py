"""HIP-graph capture of the paged, FP8 and INT8 entry points: the captured
step, replayed several times with other eager calls on the same workspace in
between, must give the eager call's bits every time (the library records no
memset nodes and keeps no state between calls), and the eager result must meet
the oracle's tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import (as_oracle_array, fp8_scale_for, int8_scale_for, make_inputs, paginate,
                                            quantize_fp8, quantize_int8)
from gpu_cases import TOL, compare, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

D = 128
SCALE = float(np.float32(1.0 / math.sqrt(D)))


def _case(kind, q_len):
    """(call(out, lse, ws, num_splits, plan), reference (out, lse), dims)."""
    lens = [3000, 700]
    q, k, v, cl = make_inputs(2, 32, 8, D, q_len, 3072, "bf16", 5000 + q_len, cache_lens=lens)
    qa = as_oracle_array(q)
    qd, cld = q.cuda(), cl.cuda()
    if kind == "paged":
        pc = paginate(k, v, cl, 16, "hnd", seed=5001)
        kd, vd, tb = pc.k_pages.cuda(), pc.v_pages.cuda(), pc.block_table.cuda()
        ref = oracle.attention(qa, as_oracle_array(k), as_oracle_array(v), cl.numpy(), SCALE)
        dims, _ = fd.paged_dims(qd, kd, tb, "hnd")

        def call(out, lse, ws, num_splits=0, plan=None):
            fd.decode_attention_paged(qd, kd, vd, tb, cld, layout="hnd", scale=SCALE, num_splits=num_splits,
                                      plan=plan, out=out, lse=lse, workspace=ws)
        return call, ref, dims, q, k, cl
    scale_for, quantize, attn, ref_fn = {
        "fp8": (fp8_scale_for, quantize_fp8, fd.decode_attention_fp8, oracle.attention_fp8),
        "int8": (int8_scale_for, quantize_int8, fd.decode_attention_int8, oracle.attention_int8),
    }[kind]
    ks, vs = scale_for(k), scale_for(v)
    kc, vc = quantize(k, ks), quantize(v, vs)
    ref = ref_fn(qa, kc.numpy(), vc.numpy(), cl.numpy(), SCALE, ks, vs)
    tb = None
    if kind == "fp8":  # FP8 through pages, INT8 contiguous
        pc = paginate(kc, vc, cl, 64, "nhd", seed=5002)
        kc, vc, tb = pc.k_pages, pc.v_pages, pc.block_table.cuda()
    kd, vd = kc.cuda(), vc.cuda()
    dims = fd.paged_dims(qd, kd, tb, "nhd")[0] if tb is not None else fd.dims_of(qd, kd)
    dims.dtype = fd.FD_BF16

    def call(out, lse, ws, num_splits=0, plan=None):
        attn(qd, kd, vd, cld, ks, vs, block_table=tb, layout="nhd", scale=SCALE, num_splits=num_splits, plan=plan,
             out=out, lse=lse, workspace=ws)
    return call, ref, dims, q, k, cl


@pytest.mark.parametrize("q_len", [1, 4, 64])
@pytest.mark.parametrize("kind", ["paged", "fp8", "int8"])
def test_graph_replays_match_eager(kind, q_len):
    say(f"[case] graph replay {kind} q_len={q_len}")
    call, ref, dims, q, k, cl = _case(kind, q_len)
    plan = fd.plan_splits(dims, cl)
    qd = q.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    ws = fd.new_workspace(max(fd.workspace_bytes(dims, max(plan.max_splits, 5)), 256), "cuda")
    call(out, lse, ws, plan=plan)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    compare(f"eager {kind}", eager_out, eager_lse, *ref, TOL["bf16"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse, ws, plan=plan)
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {rep}: out differs"
        assert torch.equal(lse, eager_lse), f"replay {rep}: lse differs"
        # eager work with another split count on the same workspace between replays
        call(torch.empty_like(out), torch.empty_like(lse), ws, num_splits=5)
        torch.cuda.synchronize()
