"""Host-side pieces of bench.py (CPU): the shader-clock readout parser, the
traffic gate, and the one-GPU guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write(tmp_path, text):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    return str(p)


def test_sclk_readout_takes_the_level_marked_current(tmp_path):
    # amdgpu lists the DPM levels one a line and marks the current one with
    # '*'; when the clock sits between levels an extra 'S:' line carries it.
    assert bench.read_sclk_mhz(write(tmp_path, "S: 98Mhz *\n0: 500Mhz\n1: 2400Mhz\n")) == 98.0
    assert bench.read_sclk_mhz(write(tmp_path, "0: 500Mhz\n1: 2400Mhz *\n")) == 2400.0
    assert bench.read_sclk_mhz(write(tmp_path, "0: 500Mhz\nS: 1801Mhz *\n1: 2400Mhz\n")) == 1801.0
    assert bench.read_sclk_mhz(write(tmp_path, "0: 500Mhz\n1: 2400Mhz\n")) is None


def test_traffic_is_reported_only_for_the_profiled_kernel(tmp_path, monkeypatch):
    # The committed counter profile carries the hash of the kernel sources
    # it was taken with; a profile of other sources gives null traffic.
    prof = tmp_path / "traffic.txt"
    prof.write_text(f"kernel_source_sha1: {bench.kernel_source_hash()}\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 123
    prof.write_text("kernel_source_sha1: 0000\nhbm_bytes_per_launch: 123\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    # A copy of the kernel sources: an edited comment or re-spaced line keeps
    # the hash (the profile still describes the kernel), an edited
    # statement changes it.
    import shutil
    src = os.path.join(ROOT, "warp_specialized_pipelined_amd", "csrc")
    dst = tmp_path / "warp_specialized_pipelined_amd" / "csrc"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.o", "_build"))
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    h0 = bench.kernel_source_hash()
    assert h0 == (monkeypatch.undo() or bench.kernel_source_hash())   # the copy hashes as the tree
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    f = dst / "kernel" / "params.hpp"
    text = f.read_text()
    f.write_text(text.replace("constexpr int kWaves = 4;",
                              "constexpr   int kWaves = 4;  // four\n/* waves */"))
    assert bench.kernel_source_hash() == h0
    f.write_text(text.replace("constexpr int kStages = 2;", "constexpr int kStages = 3;"))
    assert bench.kernel_source_hash() != h0
    assert bench.code_tokens('a = "x // y"; // z\nb;') == 'a = "x // y"; b;'


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line: nothing was measured


def test_only_the_cpu_baseline_leg_imports_the_oracle():
    """The oracle is test infrastructure: bench.py may load it for its CPU
    baseline only.  Statically, every import of it sits in cpu_baseline();
    at run time, importing bench and drawing and describing the workload
    (what the timed path does before it launches) leaves it unloaded."""
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    owners = {}
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    owners.setdefault(id(node), fn.name)
    for node in ast.walk(tree):
        names = []
        if isinstance(node, ast.Import):
            names = [a.name for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            names = [node.module or ""] + [a.name for a in node.names]
        if any(n == "oracle" or n.startswith("oracle.") or n == "oracle_operand" for n in names):
            assert owners.get(id(node)) == "cpu_baseline", (node.lineno, names)
    prog = ("import sys; sys.path.insert(0, %r); sys.argv = ['bench.py']\n"
            "import bench\n"
            "from tests.helpers import Problem\n"
            "from warp_specialized_pipelined_amd import synth\n"
            "for w in synth.WORKLOADS[:3]:\n"
            "    Problem.from_workload(w).desc()\n"
            "print('oracle' in sys.modules)\n") % ROOT
    out = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, check=True,
                         timeout=300).stdout
    assert out.strip().splitlines()[-1] == "False"
