"""The 16 x 8192x28672 + 16 x 28672x8192 workload at full size, in the launch
configuration the benchmark times (all 16 batches through muon_step_batches on
two streams, bf16 + the master of X), checked the way the benchmark checks its
first timed repetition: the two matrices with stored oracle values
(tests/golden/large_8192x28672_samples.py) at their 4096 positions (O within
the 3e-2 bar, W' within it plus the bf16 rounding of the stored W'), M'
against the momentum update, and W' and M' bitwise equal to an untimed
repeat of the same step.  Runs bench.py in a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_launch_configuration_matches_stored_oracle_samples():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py --steps 1 --warmup 0 (large workload, two streams)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0",
                        "--no-cpu-baseline", "--trace-steps", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-3000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cfg = line["config"]
    assert cfg["workload"] == "large_8192x28672" and cfg["matrices"] == 32
    assert cfg["streams"] == 2 and cfg["precision"] == "bf16_x32"
    chk = line["detail"]["check"]
    print(json.dumps(chk), flush=True)
    assert chk["reference"] == "golden" and chk["matrices"] == 2 and chk["positions_per_matrix"] == 4096
    assert chk["momentum_ok"] and chk["bitwise_as_timed"] and chk["ok"]
    assert chk["max_O_error"] <= 3e-2
    for m in chk["per_matrix"]:
        assert m["O_error"] <= 3e-2
        assert m["dW_error"] <= m["dW_allowed"]
