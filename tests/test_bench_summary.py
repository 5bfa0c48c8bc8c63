"""Host logic of bench.py's kernel-trace summary: launches between two marker
kernels are one layer's timing, in the order of the bench's per-layer rows."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _row(name, t0, dur):
    return {"Kernel_Name": name, "Start_Timestamp": str(t0), "End_Timestamp": str(t0 + dur)}


def test_layer_agreement_segments_by_marker(tmp_path, capsys):
    k1 = "void cvx::k_igemm_packed<3, 1, 1, 1>(cvx::PackedArgs)"
    k2 = "void cvx::k_stem<3, 8, 2>(cvx::StemArgs)"
    spin = "at::cuda::(anonymous namespace)::spin_kernel(long)"
    t = 0
    tr = []
    # a forward before the layer timing: not counted
    for _ in range(3):
        tr.append(_row(k1, t, 9000)); t += 10000
    plan = [("a", k1, 8000), ("s", k2, 5000), ("b", k1, 6000)]
    for _, k, d in plan:
        tr.append(_row(spin, t, 100)); t += 200
        for _ in range(4):
            tr.append(_row(k, t, d)); t += d + 50
    tr.append(_row(spin, t, 100))
    res = {"layers": [{"layer": n, "us": d / 1e3 + 0.3} for n, _, d in plan],
           "roofline": {"kernel": "cvx::k_igemm_packed<3, 1, 1, 1>", "avg_launch_us": 7.3,
                        "measured_layers": ["a", "b"]}}
    p = tmp_path / "bench.json"
    p.write_text("log line\n" + json.dumps(res) + "\n")
    bench.layer_agreement(list(reversed(tr)), str(p))  # order restored by start time
    out = capsys.readouterr().out
    # too few launches for the eager / hot graph / cold legs: all of them count
    assert "| a | `cvx::k_igemm_packed<3, 1, 1, 1>` | 4 | 8.00 | 8.00 | 8.30 |" in out
    assert "| s | `cvx::k_stem<3, 8, 2>` | 4 | 5.00 | 5.00 | 5.30 |" in out
    assert "hot graph launches 7.00 us per launch" in out


def test_layer_agreement_takes_the_hot_graph_launches(tmp_path, capsys):
    """With reps = 20: 3 + 20 eager launches, then 20 x (2 + 1) graph replays
    (hot), then the cold sets; a setup copy first does not name the layer."""
    k1 = "void cvx::k_igemm_packed<3, 1, 1, 1>(cvx::PackedArgs)"
    spin = "at::cuda::(anonymous namespace)::spin_kernel(long)"
    t = 0
    tr = [_row(spin, t, 100)]
    t += 200
    tr.append(_row("void cvx::k_copy(float*)", t, 1000)); t += 1100
    for n, d in ((23, 10000), (60, 5000), (10, 20000)):
        for _ in range(n):
            tr.append(_row(k1, t, d)); t += d + 50
    tr.append(_row(spin, t, 100))
    res = {"layer_reps": 20, "layers": [{"layer": "a", "us": 5.2}],
           "roofline": {"kernel": "cvx::k_igemm_packed<3, 1, 1, 1>", "avg_launch_us": 5.1,
                        "measured_layers": ["a"]}}
    p = tmp_path / "bench.json"
    p.write_text(json.dumps(res) + "\n")
    bench.layer_agreement(tr, str(p))
    out = capsys.readouterr().out
    allavg = (23 * 10 + 60 * 5 + 10 * 20) / 93
    assert f"| a | `cvx::k_igemm_packed<3, 1, 1, 1>` | 93 | {allavg:.2f} | 5.00 | 5.20 |" in out
    assert "hot graph launches 5.00 us per launch" in out


def test_layer_agreement_skips_on_count_mismatch(tmp_path, capsys):
    spin = "spin_kernel(long)"
    tr = [_row(spin, 0, 10), _row("void cvx::k_copy(float*)", 20, 10)]
    p = tmp_path / "bench.json"
    p.write_text(json.dumps({"layers": [{"layer": "a", "us": 1.0}, {"layer": "b", "us": 1.0}]}))
    bench.layer_agreement(tr, str(p))
    assert "layer agreement skipped" in capsys.readouterr().out
