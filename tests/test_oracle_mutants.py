"""Plant plausible mistakes in a copy of the oracle and prove the pins catch each.

Every mutant is a textual edit of ``oracle/fd_oracle.c`` compiled into a
temporary library; the real oracle is never modified.  A mutant survives only
if every pin passes, which would mean the pins cannot tell it from the oracle.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fd_oracle.c")

# (name, text in the oracle, replacement, how many occurrences to replace: 0 = all)
MUTANTS = [
    ("causal_off_by_one", "int n = L - p->q_len + t + 1;", "int n = L - p->q_len + t;", 1),
    ("causal_top_left", "int n = L - p->q_len + t + 1;", "int n = t + 1;", 1),
    ("gqa_modulo", "int g = h / (p->Hq / p->Hkv);", "int g = h % p->Hkv;", 0),
    ("scale_dropped", "return p->scale * acc;", "return acc;", 1),
    ("kv_transposed", "(((size_t)b * p->Hkv + g) * p->Lmax + j) * p->D + d",
     "(((size_t)b * p->Hkv + g) * p->D + d) * p->Lmax + j", 1),
    ("q_head_ignored", "(((size_t)b * p->Hq + h) * p->q_len + t) * p->D + d",
     "(((size_t)b * p->Hq + 0) * p->q_len + t) * p->D + d", 1),
    ("exp_sign_flipped", "Z += exp(s[j] - M);", "Z += exp(M - s[j]);", 1),
    ("weights_sign_flipped", "double w = exp(s[j] - M) / Z;", "double w = exp(M - s[j]) / Z;", 1),
    ("max_not_subtracted_in_sum", "Z += exp(s[j] - M);", "Z += exp(s[j]);", 1),
    ("lse_missing_log", "c->lse[row] = M + log(Z);", "c->lse[row] = M + Z;", 1),
    ("lse_missing_max", "c->lse[row] = M + log(Z);", "c->lse[row] = log(Z);", 1),
    ("v_from_kv_head_0", "o[d] += w * load_elem(p->v, p->dtype, kv_index(p, b, g, j, d));",
     "o[d] += w * load_elem(p->v, p->dtype, kv_index(p, b, 0, j, d));", 1),
    ("bf16_wrong_shift", "((uint32_t)x) << 16", "((uint32_t)x) << 15", 1),
    ("split_drops_tile_sum", "double wi = exp(mp[i] - mg) * li;", "double wi = exp(mp[i] - mg);", 1),
    ("split_tile_end_unclamped", "int hi = lo + T < n ? lo + T : n;", "int hi = lo + T;", 1),
    ("split_lse_is_max", "lp[i] = m + log(l);", "lp[i] = m;", 1),
    ("sequential_sum_not_rescaled", "        gsum *= diff;\n", "", 1),
    ("sequential_out_not_rescaled", "for (int d = 0; d < p->D; ++d) acc[d] *= diff;", "", 1),
    ("merge_weight_uses_max", "double w = exp(lp[i] - LSE);", "double w = exp(lp[i] - M);", 1),
    ("merge_reads_empty_slot", "            if (lp[i] == -INFINITY) continue;\n            double w",
     "            double w", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, count, tmp_path):
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found in the oracle source"
    mutated = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    assert mutated != src
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    lib = oracle.load(oracle.build(str(tmp_path / "libmutant.so"), str(c_path)))
    failures = []
    for check in ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError) as e:
            failures.append(f"{check.__name__}: {e}")
    assert failures, f"mutant {name} passed every pin"
