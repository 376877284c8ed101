"""A host model of the tile hand-off ring (CPU): tests/ring_model.cpp runs
the kernel's counting rules (csrc/kernel/handoff_rules.hpp) with threads for
waves and random delays -- the kernel's staged and overlapped schedules,
and the bare protocol with separate producer and consumer threads -- and
checks that every payload read sees its tile, that the ring never holds
more committed, unreleased tiles than it has slots (the overlapped schedule
reaching 2, the staged one staying at 1), the final counts, and that
producers block on a full ring.  Built a second time under ThreadSanitizer,
which reports any payload access the protocol's ordering fails to separate.
Planted mistakes in a copy of the rules must make it fail."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "ring_model.cpp")
KDIR = os.path.join(ROOT, "warp_specialized_pipelined_amd", "csrc", "kernel")
RULES = os.path.join(KDIR, "handoff_rules.hpp")


def build(out, include_dir, tsan=False):
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-pthread", "-I", include_dir, SRC, "-o", out]
    if tsan:
        cmd[1:1] = ["-g", "-fsanitize=thread"]
    subprocess.run(cmd, check=True)
    return out


@pytest.fixture(scope="module")
def binaries(tmp_path_factory):
    d = tmp_path_factory.mktemp("ring")
    return build(str(d / "ring_model"), KDIR), build(str(d / "ring_model_tsan"), KDIR, tsan=True)


def run(exe, mode, tiles, seed, timeout=120):
    r = subprocess.run([exe, mode, str(tiles), str(seed)], capture_output=True, text=True,
                       timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_kernel_schedules(binaries, seed):
    for mode, occ in (("staged", 1), ("overlapped", 2)):
        rc, out = run(binaries[0], mode, 300, seed)
        assert rc == 0, out
        assert f"max_occupancy={occ}" in out, out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_protocol_with_separate_producers_and_consumers(binaries, seed):
    rc, out = run(binaries[0], "split", 400, seed)
    assert rc == 0, out
    assert int(re.search(r"blocked_on_full=(\d+)", out).group(1)) > 0, out


@pytest.mark.parametrize("mode", ["staged", "overlapped", "split"])
def test_no_data_race_under_thread_sanitizer(binaries, mode):
    rc, out = run(binaries[1], mode, 150, 7, timeout=300)
    assert "ThreadSanitizer" not in out, out[-3000:]
    assert rc == 0, out


# (name, text in handoff_rules.hpp, replacement): plausible mistakes in the rules.
BROKEN_RULES = [
    ("wait_one_commit_short", "return (use + 1) * (uint32_t)kWaves;",
     "return (use + 1) * (uint32_t)kWaves - 1;"),
    ("acquire_one_release_early", "return use * (uint32_t)kWaves; }",
     "return use ? use * (uint32_t)kWaves - 1 : 0; }"),
    ("two_tiles_per_slot_use", "return (uint32_t)(n / kHandoffSlots);",
     "return (uint32_t)(n / (2 * kHandoffSlots));"),
]


@pytest.mark.parametrize("name,old,new", BROKEN_RULES, ids=[b[0] for b in BROKEN_RULES])
def test_model_catches_broken_rules(name, old, new):
    src = open(RULES).read()
    assert src.count(old) == 1, f"{name} no longer matches handoff_rules.hpp"
    with tempfile.TemporaryDirectory() as d:
        shutil.copy(os.path.join(KDIR, "params.hpp"), d)
        open(os.path.join(d, "handoff_rules.hpp"), "w").write(src.replace(old, new))
        exe = build(os.path.join(d, "ring_model"), d)
        tsan = build(os.path.join(d, "ring_model_tsan"), d, tsan=True)
        caught = []
        for seed in (1, 2, 3):
            rc, out = run(exe, "split", 2000, seed)
            caught.append(rc != 0)
        rc, out = run(tsan, "split", 300, 5, timeout=300)
        caught.append(rc != 0 or "ThreadSanitizer" in out)
    assert all(caught), (name, caught)
