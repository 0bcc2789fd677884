"""The workgroup-timeline diagnostic of the decode kernel runs and records a
consistent timeline (GPU, child process: the tool routes the binding through
its own build of the library, which the rest of the test process must not
see)."""
import json
import os
import subprocess
import sys

import pytest

from decode_attention_14_amd.build import TIMELINE_LIB

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_timeline_of_the_32k_step(cache):
    if not os.path.exists(TIMELINE_LIB):
        pytest.skip("the timeline build is made by __graft_entry__.build()")
    print(f"[case] timeline of gqa_32k over {cache} caches (child process)", flush=True)
    cmd = [sys.executable, "-m", "decode_attention_14_amd.timeline", "--launches", "2"]
    if cache == "fp8":
        cmd.append("--kv-fp8")
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-2000:])
    assert r.returncode == 0
    rows = [json.loads(ln) for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(rows) == 2
    waves = 8 if cache == "fp8" else 4
    for row in rows:
        loops = row["wave_loop_end_us"]
        assert len(loops) == waves
        # every wave leaves its loop after the first block lands and before the span ends
        assert 0 < row["first_block_us"] < min(loops) <= max(loops) < row["span_us"]
        assert 0 <= row["end_after_last_wave_us"] < row["span_us"]
        assert 0 <= row["start_spread_us"] < row["span_us"]
        # 256 workgroups over the eight XCDs
        assert sorted(int(x) for x in row["end_us_per_xcd"]) == list(range(8))
        assert 5 < row["span_us"] < 200
