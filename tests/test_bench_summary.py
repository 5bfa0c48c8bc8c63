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


def test_in_forward_table_from_the_probe_segment(tmp_path, capsys):
    """A forward probe after the per-layer segments: its launches, in plan
    order, are averaged per position and set beside each layer's hot launches
    alone; a probe whose launch count does not match the plan is skipped."""
    ka = "void cvx::k_stem_pair<2, 2, 3, true>(cvx::StemPairArgs)"
    kb = "void cvx::k_igemm_packed<3, 1, 1, 1>(cvx::PackedArgs)"
    spin = "at::cuda::(anonymous namespace)::spin_kernel(long)"
    t = 0
    tr = []
    for k, d in ((ka, 4000), (kb, 2000)):  # the two layers alone: 3 launches each
        tr.append(_row(spin, t, 10)); t += 20
        for _ in range(3):
            tr.append(_row(k, t, d)); t += d + 10
    tr.append(_row(spin, t, 10)); t += 20  # per-layer timing's last marker: the probe follows
    for _ in range(2):
        for k, d in ((ka, 5000), (kb, 3000)):
            tr.append(_row(k, t, d)); t += d + 10
    tr.append(_row(spin, t, 10))
    res = {"layer_reps": 0, "layers": [{"layer": "pre+stem", "us": 4.0}, {"layer": "bridge", "us": 2.0}],
           "forward_probe": {"forwards": 2, "launches": [["pre+stem", "cvx::k_stem_pair<2, 2, 3, true>"],
                                                         ["bridge", "cvx::k_igemm_packed<3, 1, 1, 1>"]]}}
    p = tmp_path / "bench.json"
    p.write_text(json.dumps(res) + "\n")
    bench.layer_agreement(tr, str(p))
    out = capsys.readouterr().out
    assert "| pre+stem | `cvx::k_stem_pair<2, 2, 3, true>` | 5.00 | 4.00 | 1.25 |" in out
    assert "| bridge | `cvx::k_igemm_packed<3, 1, 1, 1>` | 3.00 | 2.00 | 1.50 |" in out
    assert "| sum | | 8.00 | 6.00 | 1.33 |" in out
    res["forward_probe"]["forwards"] = 3
    p.write_text(json.dumps(res) + "\n")
    bench.layer_agreement(tr, str(p))
    assert "in-forward table skipped" in capsys.readouterr().out


def test_forward_launches_follow_the_plan():
    """One launch per plan line that is not merged into a later one, named by
    every layer it computes."""
    class L:
        def __init__(self, name):
            self.name = name

    class W:
        layers = [L("preprocess"), L("stem1"), L("stem2"), L("bridge")]

    plan = ["merged into 2", "merged into 2", "stem_pair k3 s2+s2 kernel=cvx::k_stem_pair<2, 2, 3, true> stem=1",
            "igemm_packed k3 s2 tile=0 splitk=1 kernel=cvx::k_igemm_packed<3, 1, 1, 1>"]
    assert bench.forward_launches(W, plan) == [("preprocess+stem1+stem2", "cvx::k_stem_pair<2, 2, 3, true>"),
                                               ("bridge", "cvx::k_igemm_packed<3, 1, 1, 1>")]
