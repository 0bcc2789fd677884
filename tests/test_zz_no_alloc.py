"""fd_decode_attention_noalloc (the entry point for callers that cannot
allocate) through the C ABI, against fd_decode_attention with a workspace.

The partials of the no-allocation call live in the library's static per-GPU
scratch; the kernels are those of fd_decode_attention, so the outputs must be
the same bits, and both must meet the oracle's tolerance.  Two calls in a row,
the second on a smaller input than the first (the scratch keeps the first
call's contents), then a third on yet another shape; and a call needing more
than the scratch holds fails without touching its outputs.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from decode_attention_14_amd import binding as fd
from gpu_cases import TOL, compare, inputs, run_oracle, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def _noalloc_c(qd, kd, vd, cld, sc, num_splits, plan, out, lse):
    """The raw C call (no Python-side allocation)."""
    lib = fd.load_library()
    dims = fd.dims_of(qd, kd)
    fp = plan.plan if isinstance(plan, fd.Plan) else plan
    return lib.fd_decode_attention_noalloc(ctypes.byref(dims), fd._ptr(qd), fd._ptr(kd), fd._ptr(vd), fd._ptr(cld),
                                           ctypes.c_float(sc), int(num_splits),
                                           ctypes.byref(fp) if fp is not None else None, fd._ptr(out), fd._ptr(lse),
                                           fd._stream(qd.device))


CASES = [
    # name, (B, Hq, Hkv, D, q_len, Lmax, dtype), lens, num_splits (0: planner; -n: planner for n compute
    # units, which gives these ragged batches a balanced-span plan)
    ("gqa 8k planned", (2, 32, 8, 128, 1, 8192, "bf16"), [8192, 5000], 0),
    ("smaller: mha D64 forced 5", (1, 8, 2, 64, 1, 700, "bf16"), [700], 5),
    ("chunk q_len 40 forced 3", (2, 8, 2, 128, 40, 1500, "bf16"), [1500, 300], 3),
    ("f32 forced 7", (2, 8, 2, 128, 1, 900, "f32"), [900, 31], 7),
    ("ragged, balanced spans", (5, 32, 8, 128, 1, 2000, "bf16"), [2000, 77, 0, 1500, 640], -4),
]


def test_noalloc_matches_workspace_entry_point():
    for i, (name, (B, Hq, Hkv, D, T, Lmax, dt), lens, S) in enumerate(CASES):
        say(f"[case] noalloc {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} q_len={T} Lmax={Lmax} {dt} lens={lens} S={S}")
        q, k, v, cl = inputs(B, Hq, Hkv, D, T, Lmax, dt, 7000 + i, lens)
        qd, kd, vd, cld = q.cuda(), k.cuda(), v.cuda(), cl.cuda()
        sc = _scale(D)
        plan = fd.plan_for(q, k, cl, num_cus=-S) if S < 0 else fd.plan_for(q, k, cl) if S == 0 else None
        if S < 0:
            assert plan.spans > 0
            S = 0
        ref_out, ref_lse = fd.decode_attention(qd, kd, vd, cld, scale=sc, num_splits=S, plan=plan)
        out = torch.full_like(qd, float("nan"))
        lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        st = _noalloc_c(qd, kd, vd, cld, sc, S, plan, out, lse)
        torch.cuda.synchronize()
        assert st == fd.FD_OK, fd.load_library().fd_last_error().decode()
        bits = torch.int16 if dt == "bf16" else torch.int32
        assert torch.equal(out.view(bits), ref_out.view(bits)), f"{name}: out differs from fd_decode_attention"
        assert torch.equal(lse, ref_lse), f"{name}: lse differs from fd_decode_attention"
        compare(f"noalloc {name}", out, lse, *run_oracle(q, k, v, cl, sc), TOL[dt])


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose partials need more than FD_NOALLOC_SCRATCH_BYTES fails with
    FD_ERR_WORKSPACE and leaves out and lse untouched."""
    B, Hq, Hkv, D, L = 64, 64, 8, 128, 1024
    q, k, v, cl = inputs(B, Hq, Hkv, D, 1, L, "bf16", 7100, [L] * B)
    qd, kd, vd, cld = q.cuda(), k.cuda(), v.cuda(), cl.cuda()
    need = fd.workspace_bytes(fd.dims_of(qd, kd), 256)
    assert need > fd.FD_NOALLOC_SCRATCH_BYTES
    out = torch.full_like(qd, 3.0)
    lse = torch.full(qd.shape[:3], 3.0, dtype=torch.float32, device="cuda")
    st = _noalloc_c(qd, kd, vd, cld, _scale(D), 256, None, out, lse)
    torch.cuda.synchronize()
    assert st == fd.FD_ERR_WORKSPACE
    assert "static scratch" in fd.load_library().fd_last_error().decode()
    assert bool((out == 3.0).all()) and bool((lse == 3.0).all())
