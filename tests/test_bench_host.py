"""Host-side checks of bench.py's helpers (no GPU): the one-GPU refusal, the
selection counts of a step from its masks, and the rule that counter
traffic is reported only for the kernel sources it was measured on."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def _mask(bits, W, n_c):
    """[W][ceil(n_c/32)] int32 mask with bit c of worker w set for (w, c) in bits."""
    import torch
    mw = (n_c + 31) // 32
    m = np.zeros((W, mw), np.uint32)
    for w, c in bits:
        m[w, c // 32] |= np.uint32(1) << np.uint32(c % 32)
    return torch.from_numpy(m.view(np.int32))


def test_selection_stats_brute_force():
    """Counts against a direct loop over (worker, chunk), with chunks past bit
    31 of a word."""
    rng = np.random.default_rng(5)
    W, C, n_c = 3, 256, 70
    P = (n_c - 1) * C + 77
    plan = types.SimpleNamespace(n_chunks=n_c, chunk=C)
    prev = {(w, c) for w in range(W) for c in range(n_c) if rng.random() < 0.3}
    cur = {(w, c) for w in range(W) for c in range(n_c) if rng.random() < 0.3}
    prev |= {(0, n_c - 1)}
    cur |= {(0, n_c - 1), (1, n_c - 1)}
    got = bench.selection_stats(plan, _mask(prev, W, n_c), _mask(cur, W, n_c), P)
    assert got["pairs_sent"] == len(cur)
    assert got["pairs_sent_again"] == len(prev & cur)
    assert got["pairs_newly_sent"] == len(cur - prev)
    assert got["chunks_sent_by_any_worker"] == len({c for _, c in cur})
    assert bench.selection_stats(plan, None, _mask(cur, W, n_c), P)["pairs_newly_sent"] == len(cur)


def test_traffic_needs_the_profiled_code(tmp_path):
    """A counter record is returned while the code of its sources is the code
    it was measured on (comments and blank lines aside), and not once the code
    changes or a source is missing."""
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n    return x + 1;  // v1\n}\n")
    rel = os.path.relpath(str(src), bench.ROOT)
    rec = {"k_x": {"bytes_per_launch": 123, "sources": [rel], "code_sha256": bench.code_digest([src.read_text()]),
                   "summary": "s.md"}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(path), "k_x")["bytes_per_launch"] == 123
    assert bench.measured_traffic(str(path), "k_other") is None
    src.write_text("/* the kernel,\n   described */\nint f(int x) {\n\n    return x + 1;  // v2\n}\n")
    assert bench.measured_traffic(str(path), "k_x")["bytes_per_launch"] == 123
    src.write_text("int f(int x) {\n    return x + 2;  // v1\n}\n")
    assert bench.measured_traffic(str(path), "k_x") is None
    src.unlink()
    assert bench.measured_traffic(str(path), "k_x") is None
    assert bench.measured_traffic(str(tmp_path / "absent.json"), "k_x") is None


@pytest.mark.parametrize("name", sorted(f[len("traffic_"):-len(".json")] for f in os.listdir(os.path.join(ROOT, "profiles"))
                                         if f.startswith("traffic_") and f.endswith(".json")))
def test_committed_traffic_matches_current_sources(name):
    """Every committed counter record still describes the kernel sources in
    the tree, so bench.py reports its traffic."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    with open(path) as f:
        keys = list(json.load(f))
    assert keys
    for k in keys:
        assert bench.measured_traffic(path, k) is not None, (name, k)
