"""The host planner built on its own with the address and undefined-behaviour
sanitizers (g++, host code only), run over random and edge-case offsets:
no sanitizer report, and the same words as the planner oracle."""

import os
import random
import shutil
import subprocess

import pytest

from oracle.planner_ref import plan_words_ref, workspace_bound_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cases():
    rng = random.Random(7)
    cases = [
        (1, [0]),
        (8, [5, 5, 5]),
        (2, [0, 300, 300, 700]),
        (2, [0, 3000, 3200, 3300, 4000]),
        (256, [8192 * i for i in range(257)]),
        (256, [0, 65536]),
        (1, [0, 2 ** 30, 2 ** 31 - 1]),
        (256, [5, 2 ** 31 - 1]),
        (3, [0, 1, 2 ** 31 - 2, 2 ** 31 - 1]),
    ]
    for _ in range(300):
        n = rng.randint(0, 60)
        ind = [rng.choice([0, rng.randint(0, 10 ** 6)])]
        for _ in range(n):
            ind.append(ind[-1] + rng.choice([0, 1, rng.randint(0, 300), rng.randint(0, 20000),
                                             rng.randint(0, 200000)]))
        cases.append((rng.choice([1, 2, 3, 7, 64, 256, 304]), ind))
    return cases


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "plan_harness")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "plan_harness.cpp"),
           os.path.join(ROOT, "mla_mxfp4_kv_amd", "csrc", "mla_plan.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail("sanitizer build failed:\n" + res.stderr[-3000:])
    return out


def test_planner_under_sanitizers_matches_oracle(harness):
    cases = _cases()
    text = "".join(f"{cus} {len(ind) - 1} {' '.join(map(str, ind))}\n" for cus, ind in cases)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([harness], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    lines = res.stdout.splitlines()
    assert len(lines) == len(cases)
    for (cus, ind), line in zip(cases, lines):
        words, need = plan_words_ref(ind, len(ind) - 1, cus)
        f = line.split()
        assert f[0] == "need" and f[2] == "bound" and f[4] == "words", line[:80]
        assert int(f[1]) == need
        assert int(f[3]) == workspace_bound_ref(len(ind) - 1, ind[-1] - ind[0], cus)
        assert [int(x) for x in f[5:]] == words, (cus, ind[:5])


def test_planner_under_sanitizers_refuses_bad_offsets(harness):
    text = "4 2 0 5 3\n4 1 -1 5\n0 1 0 5\n"
    res = subprocess.run([harness], input=text, capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr[-3000:]
    assert res.stdout.split("\n")[:3] == ["error -1", "error -1", "error -1"]
