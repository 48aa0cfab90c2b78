"""bench.py's host-side contract (no GPU): it measures one GPU and refuses
--gpus N > 1 with a message, and the HBM traffic it reports comes from a
profile summary only while the kernel sources still hash to the recorded
SHA-256."""

import hashlib
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _write_profile(root, kernel, workload, sources, traffic):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(root, f), "rb").read())
    rec = {"kernel": kernel, "workload": workload, "source_files": sources,
           "source_sha256": h.hexdigest(), "traffic_bytes_per_launch": traffic}
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"{kernel}__{workload}.md"), "w") as fh:
        fh.write(f"# summary\n\n```json traffic\n{json.dumps(rec)}\n```\n")


def test_traffic_only_while_sources_match(tmp_path):
    bench = _bench_module()
    root = str(tmp_path)
    os.makedirs(os.path.join(root, "src"))
    for name, text in (("a.hip", "kernel a\n"), ("b.h", "header b\n")):
        with open(os.path.join(root, "src", name), "w") as fh:
            fh.write(text)
    _write_profile(root, "k", "w", ["src/a.hip", "src/b.h"], 123456)
    bench.ROOT = root
    assert bench.recorded_traffic("k", "w") == 123456
    assert bench.recorded_traffic("k", "other") is None          # no summary
    with open(os.path.join(root, "src", "b.h"), "a") as fh:      # a source changed
        fh.write("// edit\n")
    assert bench.recorded_traffic("k", "w") is None


def test_committed_summaries_name_existing_sources():
    # Every committed summary records its command and the source files its
    # hash covers, and those files exist.
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith(".md")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "rocprofv3 --kernel-trace --stats" in text and "--pmc FETCH_SIZE" in text, n
        rec = json.loads(text.split("```json traffic", 1)[1].split("```", 1)[0])
        kernel, workload = n[:-3].split("__")
        assert rec["kernel"].startswith(kernel) and rec["workload"] == workload, n
        for f in rec["source_files"]:
            assert os.path.exists(os.path.join(ROOT, f)), (n, f)
