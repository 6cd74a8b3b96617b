"""The oracle still reproduces its committed tiny trajectory bit for bit."""
import importlib.util
import json
import os


def test_oracle_reproduces_golden_trajectory(root):
    gdir = os.path.join(root, "tests", "golden")
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(gdir, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(gdir, "oracle_tiny_trajectory.json")) as f:
        stored = json.load(f)
    assert mod.trajectory() == stored
