"""CPU checks of bench.py's command-line contract (no GPU needed): it runs on
one GPU only and says so for any other count, and it names the workload and
the fields the JSON line carries."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2", "--no-cpu-baseline")
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in rec["error"] and rec["requested_gpus"] == 2


def test_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--settle-ms", "--no-cpu-baseline"):
        assert flag in r.stdout


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path):
    """bench.traffic() returns the stored bytes while the kernel source's code
    hash (comments and blank space removed) matches, and None otherwise."""
    sys.path.insert(0, ROOT)
    import bench
    for src, (h, rows) in bench.TRAFFIC.items():
        path = os.path.join(ROOT, "whisper_attention_amd", "csrc", src)
        current = bench.code_hash(path) == h
        for launch, val in rows.items():
            assert bench.traffic(src, launch) == (val if current else None)
    # a comment-only edit keeps the hash; a code edit changes it
    src = open(os.path.join(ROOT, "whisper_attention_amd", "csrc", "kv_dequant.hip")).read()
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text(src)
    b.write_text("// another comment\n" + src.replace("\n", "\n\n", 3))
    c.write_text(src + "\nstatic int unused_counter = 1;\n")
    assert bench.code_hash(str(a)) == bench.code_hash(str(b)) != bench.code_hash(str(c))
