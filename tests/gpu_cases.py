"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, then compare element by element.

Tolerances: max abs error 2e-3 for bf16 inputs (fp32 accumulation) and 1e-5
for fp32 inputs, on out and on lse.  A bf16 out is also rounded to bf16 (RNE,
half an ulp = 2^-9 of the value): where |out| is O(1) -- a handful of keys --
that rounding alone exceeds 2e-3, so bf16 outputs get 2e-3 plus one bf16 ulp
of the reference value (2^-8 |ref|; half an ulp for the rounding, half for a
fp32 result within fp32 error of a rounding midpoint).  At the benchmark
workloads |out| < 0.25, so compare_workload asserts the flat 2e-3 there, with
no ulp allowance, plus a rel-L2 regression guard.
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


# rel-L2 guard at the workloads: ||out - r|| / ||r||, r = the oracle's output
# rounded to out's dtype.  Rounding the GPU's fp32 result to bf16 flips a
# rounding only where it lies within its own error of a midpoint, so with
# fp32-accurate arithmetic this stays near 1e-4; the fp64 values themselves
# sit about 2^-9 / sqrt(3) ~ 1.1e-3 (relative rms) from their bf16 roundings,
# which is why the guard is taken against r and not against the fp64 output.
#
# That holds for the decode kernel (up to 32 query rows per KV head), which
# feeds P to the P.V product as a bf16 head plus a bf16 remainder (about 16
# significant bits).  The chunk kernel (more rows per KV head) feeds P as one
# bf16 operand, as matrix-core attention usually does, except in blocks where
# one key carries more than 1/16 of the running sum: each weight then carries
# a relative rounding error of rms 2^-9 / sqrt(3) ~ 1.1e-3, which reaches the
# output at about the same relative rms, comparable to half a bf16 ulp of the
# output; the rounded result then differs from the rounded oracle by one ulp
# (2^-8 relative) at roughly E|err| / ulp ~ 23% of the elements, a rel-L2 of
# about sqrt(0.23) 2^-8 ~ 1.9e-3.  Its guard is REL_L2_GUARD_CHUNK.
REL_L2_GUARD = 1e-3
REL_L2_GUARD_CHUNK = 3e-3


def rel_l2_rounded(got_out, ref_out):
    """rel-L2 of out against the oracle output rounded to out's dtype (RNE)."""
    r = torch.from_numpy(np.ascontiguousarray(ref_out)).to(got_out.dtype).double().numpy()
    g = got_out.detach().cpu().double().numpy()
    den = float(np.linalg.norm(r))
    return float(np.linalg.norm(g - r)) / den if den > 0 else float(np.linalg.norm(g))


def rel_l2_guard_for(rows_per_kv_head):
    """The rel-L2 guard of the kernel that serves a call with this many query
    rows per KV head (n_rep * q_len): the decode kernel up to 32, else the
    chunk kernel."""
    return REL_L2_GUARD if rows_per_kv_head <= 32 else REL_L2_GUARD_CHUNK


def compare_workload(name, got_out, got_lse, ref_out, ref_lse, guard=REL_L2_GUARD):
    """Check at a benchmark workload's shape: max abs error <= 2e-3 (bf16) or
    1e-5 (fp32) on out and on lse with no ulp allowance, and rel-L2 of out
    against the rounded oracle <= guard.  Returns (max abs error of out, of
    lse, rel-L2)."""
    tol = TOL["bf16"] if got_out.dtype == torch.bfloat16 else TOL["f32"]
    go = got_out.detach().float().cpu().numpy().astype(np.float64)
    assert go.shape == ref_out.shape, (name, go.shape, ref_out.shape)
    assert not np.isnan(go).any(), f"{name}: NaN in out"
    err = float(np.max(np.abs(go - ref_out))) if go.size else 0.0
    assert err <= tol, f"{name}: out max abs error {err:.3e} > {tol:.1e}"
    gl = got_lse.detach().float().cpu().numpy().astype(np.float64)
    inf_r = np.isinf(ref_lse)
    assert np.array_equal(np.isinf(gl), inf_r), f"{name}: lse infinities differ"
    fin = ~inf_r
    lerr = float(np.max(np.abs(gl[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert lerr <= tol, f"{name}: lse max abs error {lerr:.3e} > {tol:.1e}"
    rl2 = rel_l2_rounded(got_out, ref_out)
    say(f"  {name}: max abs err out {err:.2e} lse {lerr:.2e}; rel-L2 vs rounded oracle {rl2:.2e} "
        f"(max |out| {float(np.max(np.abs(ref_out))):.3f})")
    assert rl2 <= guard, f"{name}: rel-L2 {rl2:.3e} above the guard {guard:.0e}"
    return err, lerr, rl2


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
