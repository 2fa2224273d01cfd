"""The split-KV planner built host-only with AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp has no HIP dependency, so g++ builds it with the sanitizers beside a small
driver (tests/native/plan_driver.cpp); the driver's plans for random and edge-case
batches must equal the oracle's (oracle/plan.py) element by element, and any
out-of-bounds access, leak, signed overflow or other undefined behaviour aborts the
driver (-fno-sanitize-recover), which fails the test.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import plan as PL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_decode_03_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan_asan") / "plan_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def run_cases(exe, cases):
    text = "".join(f"{B} {Sq} {N} {C}\n" + " ".join(str(int(x)) for x in L) + "\n"
                   for (L, Sq, N, C, B) in cases)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    out, i = [], 0
    for _ in cases:
        head = lines[i].split()
        i += 1
        if head[0] == "err":
            out.append(None)
            continue
        nparts, npartials, nitems, nred = map(int, head[1:])
        items = [tuple(map(int, lines[i + k].split())) for k in range(nitems)]
        i += nitems
        red = [tuple(map(int, lines[i + k].split())) for k in range(nred)]
        i += nred
        out.append(dict(items=items, reduce=red, num_parts=nparts, num_partials=npartials))
    assert i == len(lines)
    return out


def test_sanitized_plans_equal_oracle(driver):
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(150):
        B = int(rng.integers(1, 300))
        Sq = int(rng.integers(1, 9))
        N = int(rng.integers(1, 129))
        C = int(rng.integers(1, 400))
        hi = int(rng.choice([64, 1000, 20000, 200000]))
        L = rng.integers(0, hi, size=B)
        cases.append((L, Sq, N, C, B))
    # edge cases: empty requests, one key, granule boundaries, one CU, the largest seq_len
    cases += [([0], 1, 1, 1, 1), ([0, 0, 0], 4, 128, 256, 3), ([1], 1, 128, 256, 1),
              ([63, 64, 65, 127, 128, 129], 1, 16, 3, 6), ([1 << 30], 1, 128, 256, 1),
              ([1 << 30, 5, (1 << 30) - 1], 8, 128, 304, 3), ([4096] * 32, 4, 128, 256, 32)]
    got = run_cases(driver, cases)
    for (L, Sq, N, C, B), g in zip(cases, got):
        ref = PL.split_plan(L, Sq, N, C)
        assert g is not None, (list(L)[:8], Sq, N, C)
        assert g["items"] == [tuple(x) for x in ref["items"]]
        assert g["reduce"] == [tuple(x) for x in ref["reduce"]]
        assert g["num_parts"] == ref["num_parts"] and g["num_partials"] == ref["num_partials"]


def test_sanitized_plan_rejects_bad_input(driver):
    got = run_cases(driver, [([-1], 1, 1, 4, 1), ([(1 << 30) + 1], 1, 1, 4, 1), ([2 ** 31 - 1], 1, 128, 256, 1),
                             ([5], 0, 1, 4, 1), ([5], 1, 1, 0, 1)])
    assert all(g is None for g in got)
