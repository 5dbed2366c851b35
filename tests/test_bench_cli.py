"""bench.py on the CPU: the single-GPU refusal and the workload list (no GPU needed)."""
import json
import os
import subprocess
import sys

import synth_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_configs_cover_every_workload_family():
    """Every workload the benchmark names besides the N sweep is timed, with the P.V mode's
    ceiling: FP16 P.V halves the rate of half the work (2/3), D96 padded to 128 loses a
    quarter more (1/2)."""
    fams = {(fam, tuple(sorted(kw.items()))): ceil for _, fam, kw, ceil in bench.CONFIGS}
    assert set(f for f, _ in fams) == {"tiny", "llm_prefill", "video_dit", "gqa"}
    assert fams[("llm_prefill", ())] == 2 / 3 and fams[("llm_prefill", (("causal", True),))] == 2 / 3
    assert fams[("video_dit", ())] == 1.0
    assert fams[("gqa", ())] == 2 / 3 and fams[("gqa", (("D", 96),))] == 0.5
    for label, fam, kw, _ in bench.CONFIGS:
        w = si.workload(fam, **kw)
        assert f"N{w.Nq}" in label and f"D{w.D}" in label and w.layout in label
        assert ("causal" in label.split()) == bool(w.causal) or ("non-causal" in label) == (not w.causal)
