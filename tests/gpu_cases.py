"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, then compare element by element.

Tolerances: max abs error 2e-3 for bf16 inputs (fp32 accumulation) and 1e-5
for fp32 inputs, on out and on lse.  A bf16 out is also rounded to bf16 (RNE,
half an ulp = 2^-9 of the value): where |out| is O(1) -- a handful of keys --
that rounding alone exceeds 2e-3, so bf16 outputs get 2e-3 plus one bf16 ulp
of the reference value (2^-8 |ref|; half an ulp for the rounding, half for a
fp32 result within fp32 error of a rounding midpoint).  At the benchmark
workloads |out| < 0.25 and the extra term stays below 1e-3.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from decode_attention_14_amd import binding as fd
from decode_attention_14_amd.inputs import as_oracle_array, make_inputs

TOL = {"bf16": 2e-3, "f32": 1e-5}
BF16_OUT_REL = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare(name, got_out, got_lse, ref_out, ref_lse, tol):
    """Element-wise check; returns (max abs error of out, of lse)."""
    go = got_out.detach().float().cpu().numpy().astype(np.float64)
    gl = got_lse.detach().float().cpu().numpy().astype(np.float64)
    assert go.shape == ref_out.shape, (name, go.shape, ref_out.shape)
    assert not np.isnan(go).any(), f"{name}: NaN in out"
    bound = tol + (BF16_OUT_REL * np.abs(ref_out) if got_out.dtype == torch.bfloat16 else 0.0)
    diff = np.abs(go - ref_out)
    err = float(np.max(diff)) if go.size else 0.0
    worst = float(np.max(diff - bound)) if go.size else -1.0
    assert worst <= 0, f"{name}: out error exceeds bound by {worst:.3e} (max abs error {err:.3e})"
    inf_r = np.isinf(ref_lse)
    assert np.array_equal(np.isinf(gl), inf_r), f"{name}: lse infinities differ"
    assert np.all(gl[inf_r] == ref_lse[inf_r]), f"{name}: lse -inf sign"
    fin = ~inf_r
    lerr = float(np.max(np.abs(gl[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert lerr <= tol, f"{name}: lse max abs error {lerr:.3e} > {tol:.1e}"
    return err, lerr


def inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, lens, q_mul=1.0, poison=False):
    q, k, v, cl = make_inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, cache_lens=lens)
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(q.dtype)
    if poison:
        for b, L in enumerate(cl.tolist()):
            k[b, :, L:] = float("nan")
            v[b, :, L:] = float("inf")
    return q, k, v, cl


def run_gpu(q, k, v, cl, scale, num_splits=0, plan=None, device="cuda"):
    qd, kd, vd, cld = (t.to(device) for t in (q, k, v, cl))
    out, lse = fd.decode_attention(qd, kd, vd, cld, scale=scale, num_splits=num_splits, plan=plan)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(q, k, v, cl, scale):
    return oracle.attention(as_oracle_array(q), as_oracle_array(k), as_oracle_array(v),
                            cl.numpy(), scale)


def check_case(name, B, Hq, Hkv, D, T, Lmax, dt, seed, lens, num_splits=0, use_plan=False,
               q_mul=1.0, poison=False, scale=None):
    say(f"[case] {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} q_len={T} Lmax={Lmax} {dt} "
        f"lens={lens if len(lens) <= 8 else str(lens[:8]) + '...'} splits={num_splits} plan={use_plan}")
    q, k, v, cl = inputs(B, Hq, Hkv, D, T, Lmax, dt, seed, lens, q_mul, poison)
    scale = float(np.float32(1.0 / math.sqrt(D))) if scale is None else float(np.float32(scale))
    plan = fd.plan_for(q, k, cl, num_splits=0) if use_plan else None
    ref_out, ref_lse = run_oracle(q, k, v, cl, scale)
    out, lse = run_gpu(q, k, v, cl, scale, num_splits, plan)
    return compare(name, out, lse, ref_out, ref_lse, TOL[dt])
