"""Step plans run on host threads under ThreadSanitizer.

tests/plan_executor.cpp walks every workgroup's task list on its own thread
the way the persistent kernel does (claim pools included), waiting on
counters with acquire loads and signalling with release adds, and checks
each read against the tasks that produce it (the read relation the plan
validator proves covered). A read that no chain of waits orders after its
producer is a data race, whatever the timing, so these runs check the
counter protocol of the pages' design (per-tile counters recording when a
task's inputs are ready: "Cohere Publishes One-Kernel Server for North Mini
Code, Claims 1.58x vLLM Speedup", "One resident program, many small tasks")
on real plans, not only the plan's static invariants. ThreadSanitizer keeps only a few accesses per 8 bytes and
can lose one to other threads' reads, so the executor also carries a vector
clock through the waits and signals and reports an unordered read on every
run: planted missing waits must be reported by it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "persistent_megakernel_03_amd", "csrc")

# op codes of the task records
OP_ATTN, OP_COMBINE, OP_OPROJ, OP_ROUTER, OP_DOWN, OP_LMHEAD = 2, 3, 4, 5, 8, 10


@pytest.fixture(scope="module")
def executor(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("plan_executor") / "plan_executor")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "plan_executor.cpp"), os.path.join(CSRC, "mk_plan.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(exe, shape, n_wg, positions, shared_levels, seed, drop_op=None):
    args = [exe, shape, str(n_wg), ",".join(str(p) for p in positions), str(shared_levels), str(seed)]
    if drop_op is not None:
        args.append(str(drop_op))
    env = dict(os.environ, TSAN_OPTIONS="exitcode=66 second_deadlock_stack=1")
    return subprocess.run(args, capture_output=True, text=True, timeout=600, env=env)


def _positions(n, lo, hi, step):
    return [lo + (i * step) % (hi - lo) for i in range(n)]


CLEAN = [
    ("tiny", 8, [5], 0),
    ("tiny", 16, [5, 9, 33], 0),
    ("tiny", 16, [5, 9, 33, 70], 1),
    ("tiny", 24, [1, 100, 700, 3], 2),
    ("tiny", 64, _positions(20, 1, 900, 131), 0),
    ("tiny", 12, [64, 64, 64], -1),
    ("a3b", 512, [8191], 0),
    ("a3b", 512, [8191, 100], 0),
    ("a3b", 512, [5, 900, 3000], 0),
    ("a3b", 512, _positions(64, 50, 8050, 977), 2),
]


@pytest.mark.parametrize("shape,n_wg,positions,shared", CLEAN,
                         ids=[f"{c[0]}-wg{c[1]}-b{len(c[2])}-s{c[3]}" for c in CLEAN])
def test_plan_runs_race_free(executor, shape, n_wg, positions, shared):
    r = _run(executor, shape, n_wg, positions, shared, seed=len(positions))
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-6000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.startswith("ok tasks"), r.stdout


# Each case takes the main wait away from the first task of one op in layer
# 0 whose producers run on other workgroups (where the task's own workgroup
# ran its producers, program order still covers the read and nothing is
# missing).
PLANTED = [
    ("tiny", 8, [5], 0, OP_ATTN),
    ("tiny", 8, [5], 0, OP_COMBINE),
    ("tiny", 8, [5], 0, OP_OPROJ),
    ("tiny", 8, [5], 0, OP_ROUTER),
    ("tiny", 16, [5, 9, 33, 70], 0, OP_COMBINE),
    ("tiny", 16, [5, 9, 33, 70], 0, OP_DOWN),
    ("tiny", 16, [5, 9, 33, 70], 0, OP_LMHEAD),
    ("tiny", 24, [1, 100, 700, 3], 2, OP_OPROJ),   # a task claimed from a pool
    ("a3b", 512, [4000], 0, OP_DOWN),
]


@pytest.mark.parametrize("seed", [3, 7])
@pytest.mark.parametrize("shape,n_wg,positions,shared,drop_op", PLANTED,
                         ids=[f"{c[0]}-b{len(c[2])}-s{c[3]}-op{c[4]}" for c in PLANTED])
def test_missing_wait_is_reported(executor, shape, n_wg, positions, shared, drop_op, seed):
    r = _run(executor, shape, n_wg, positions, shared, seed=seed, drop_op=drop_op)
    assert r.returncode != 0, r.stdout
    assert "which no wait orders before it" in r.stdout or "before it was written" in r.stdout, \
        r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("shape,n_wg,positions", [("tiny", 16, [5, 9, 33, 70]), ("a3b", 512, [4000])],
                         ids=["tiny-b4", "a3b-b1"])
def test_never_satisfied_counter_times_out(executor, shape, n_wg, positions):
    # the first waiting task of layer 0 waits for one signal more than its
    # counter ever gets: every thread must give up at the deadline, no hang
    args = [executor, shape, str(n_wg), ",".join(map(str, positions)), "0", "1", "stuck", "2"]
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0, r.stdout
    assert "deadlock: counter" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
