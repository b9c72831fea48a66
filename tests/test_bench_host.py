"""bench.py and the product sources on the host: the one-GPU contract and where the oracle may enter."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a refused run


def test_oracle_is_imported_only_by_the_cpu_baseline_legs():
    tree = ast.parse(open(BENCH).read())
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any("oracle" in ast.dump(n) for n in top), "bench.py imports the oracle at module level"
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for n in ast.walk(fn):
                if isinstance(n, (ast.Import, ast.ImportFrom)) and "oracle" in ast.dump(n):
                    users.add(fn.name)
    assert users and all(u.startswith("cpu_baseline") for u in users), users


def test_product_sources_never_reference_the_oracle():
    """The library, its headers and the binding stand alone: no file of the product path names the
    oracle, so no step can route through it."""
    hits = []
    for base in ("token_dispatch_grouped_route_amd", "include"):
        for dirpath, _, files in os.walk(os.path.join(ROOT, base)):
            for f in files:
                if f.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                    path = os.path.join(dirpath, f)
                    if "oracle" in open(path, errors="replace").read():
                        hits.append(os.path.relpath(path, ROOT))
    assert not hits, hits


def test_training_step_cpu_baseline_runs_on_a_small_workload():
    """The training step's CPU baseline leg end to end on a reduced wide-expert share: a positive
    rate, the host's thread count, and a sample no larger than the workload."""
    sys.path.insert(0, ROOT)
    import bench
    import moe_workloads as mw
    w = mw.scaled(mw.get("wide_share_fwd_bwd"), T=96, H=128, I=64, E=16, EL=8, k=4)
    r = bench.cpu_baseline_bwd(w, mw.inputs(w, 0), budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    n_tok = int(r["sample"].split(" of ")[1].split()[-1])
    assert 1 <= n_tok <= w.T
