"""The persistent kernel's inter-tile protocol, and the one-tile kernel's two-level
look-back, run on the CPU (tests/protocol_model/pipeline_model.cpp: one thread per
wavefront, random pauses at every step, workgroups starting late and in any order),
also under ThreadSanitizer.

The lecture points out that a scan whose blocks pass carries to each other inside
one kernel depends on how their memory accesses are ordered and on blocks busy-waiting
for one another, and that a race there shows up as results that differ between runs
([L7] concept 6 "层次化扫描（Hierarchical Scan）"; "常见陷阱与注意事项").  These tests
run thousands of schedules the GPU cannot be made to show on demand and check, on
every run, the outputs against a sequential scan, that no wait gave up, that the
launch's counters were reset for the next one, and (under ThreadSanitizer) that every
access to the LDS rings is ordered by the protocol.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol_model", "pipeline_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("protocol_model")
    plain, tsan = str(d / "pm"), str(d / "pm_tsan")
    subprocess.run([gxx, "-O2", "-std=c++17", "-pthread", "-Wall", "-Werror", SRC, "-o", plain], check=True)
    r = subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=thread", SRC, "-o", tsan],
                       capture_output=True, text=True)
    return {"plain": plain, "tsan": tsan if r.returncode == 0 else None}


def run(binary, timeout=120, **kw):
    args = [binary] + ["%s=%s" % (k, v) for k, v in kw.items()]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0 report_signal_unsafe=0")
    p = subprocess.run(args, capture_output=True, text=True, timeout=timeout, env=env)
    line = [l for l in p.stdout.splitlines() if l.startswith("result")]
    assert line, "no result line: %s %s" % (p.stdout, p.stderr[-2000:])
    fields = dict(f.split("=") for f in line[0].split()[1:])
    return p.returncode, fields, p.stderr


# (data waves, tiles waiting per wave, resolver span, operator 0 add / 1 affine): the
# pipeline depths and resolver windows (tiles waiting / tiles per lane of a window)
# of the shipped classes -- plain scans and affine maps 3/1, segmented 2/2,
# compaction 3/1, (maximum, count) 3/2, 2x2 matrices 4/4,
# 3x3 matrices 1/2 -- with one-word and two-word carries
SHIPPED = [(3, 3, 1, 1), (3, 3, 1, 0), (5, 2, 2, 1), (3, 4, 1, 0), (2, 3, 4, 1), (1, 2, 2, 0), (4, 1, 1, 1),
           (2, 3, 2, 1), (3, 4, 4, 1), (2, 1, 2, 1)]


@pytest.mark.parametrize("nd,wait,span,op", SHIPPED)
def test_persistent_pipeline_random_schedules(model, nd, wait, span, op):
    # first tile numbers as one batch, and (the plain scans, affine maps, 2x2
    # matrices) as a piece of one, then pieces of three
    for seed, first in ((1, 1), (2, 0), (3, 1)):
        rc, f, err = run(model["plain"], nd=nd, wait=wait, span=span, op=op, seed=seed, tiles=300, wgs=5,
                         launches=3, first_piece=first)
        assert rc == 0 and f["ok"] == "1", (f, err[-1000:])
        assert f["mismatches"] == "0" and f["err"] == "0"


def test_persistent_pipeline_many_workgroups_and_no_pauses(model):
    rc, f, err = run(model["plain"], nd=3, wait=3, wgs=17, tiles=1500, seed=7, delay=0, launches=4)
    assert rc == 0 and f["ok"] == "1", (f, err[-1000:])
    rc, f, err = run(model["plain"], nd=2, wait=3, wgs=3, tiles=700, seed=8, delay=600, launches=2)
    assert rc == 0 and f["ok"] == "1", (f, err[-1000:])


def test_epoch_wrap(model):
    # launches 4094, 4095, then the wrap to 1 (the status words are cleared), then 2
    rc, f, err = run(model["plain"], epoch_start=4094, launches=4, tiles=200, seed=11)
    assert rc == 0 and f["ok"] == "1", (f, err[-1000:])
    rc, f, err = run(model["plain"], kernel=1, epoch_start=4094, launches=4, tiles=200, seed=12)
    assert rc == 0 and f["ok"] == "1", (f, err[-1000:])


@pytest.mark.parametrize("op", [0, 1])
def test_one_tile_kernel_two_level_lookback(model, op):
    # 100 tiles: the second group folds the first group's tile words; 300 tiles: within
    # five groups; 4200 tiles: more than 64 groups, so the walk over the groups takes a
    # second window
    for seed, tiles in ((4, 100), (1, 300), (2, 300), (3, 4200)):
        rc, f, err = run(model["plain"], kernel=1, op=op, tiles=tiles, seed=seed, launches=2,
                         delay=200 if tiles < 1000 else 20, timeout=300)
        assert rc == 0 and f["ok"] == "1", (f, err[-1000:])


def test_ring_needs_twice_the_wait_plus_one(model):
    """The slot ring (arrivals, wave totals, prefixes) must hold 2 * WAIT + 1 uses: a data
    wave hands over tile k + WAIT - 1 in iteration k, but the first batch hands over its
    WAIT + 1 tiles before iteration 0, so with 2 * WAIT slots a fast wave can hand over a
    tile into a slot whose previous tile a slow wave has not read yet (stale wave totals,
    or an arrival counted for the wrong tile and a total never published).  The kernel's
    16 slots hold the shipped depths (WAIT <= 4); WAIT = 8 would not."""
    for wait in (2, 3, 4):
        for seed in range(1, 5):
            # the default budget: with the short one below, a wait descheduled by the host can
            # give up, and a wave that gave up reads whatever its slot holds
            rc, f, err = run(model["plain"], wait=wait, slots=2 * wait + 1, tiles=240, seed=seed)
            assert rc == 0 and f["ok"] == "1", ("2*WAIT+1 slots", wait, f, err[-1000:])
        failed = False
        for seed in range(1, 60):
            rc, f, err = run(model["plain"], wait=wait, slots=2 * wait, tiles=240, seed=seed, spin=20000)
            if rc != 0:
                assert "stale" in err or f["err"] != "0" or f["mismatches"] != "0"
                failed = True
                break
        assert failed, "2*WAIT slots never failed for WAIT=%d" % wait


@pytest.mark.parametrize("kernel", [0, 1])
def test_lost_total_ends_the_launch(model, kernel):
    """A tile whose total is never published: every wait is bounded, the launch ends and
    reports the timeout; with the abort word (sticky give-ups) it ends sooner than with
    budgets restarted per window and per tile."""
    spent = {0: [], 1: []}  # waits that polled their whole budget
    for seed in (3, 4, 5):
        for sticky in (1, 0):
            rc, f, err = run(model["plain"], kernel=kernel, lose_tile=37, sticky=sticky, spin=100000, seed=seed,
                             tiles=300, timeout=300)
            assert rc == 0 and f["ok"] == "1" and int(f["err"]) & 1, (f, err[-1000:])
            spent[sticky].append(int(f["full_budgets"]))
    # sticky: the first give-up ends the others' waits at their next check
    assert all(1 <= c <= 2 for c in spent[1]), spent
    # restarted budgets: a whole budget per window or per waiting tile
    assert max(spent[0]) > 2, spent


def test_thread_sanitizer_finds_no_race(model):
    if model["tsan"] is None:
        pytest.skip("ThreadSanitizer build not available")
    for kw in (dict(nd=3, wait=3, span=1, op=1, seed=1), dict(nd=2, wait=1, span=2, op=0, seed=2),
               dict(nd=4, wait=4, span=4, op=1, seed=3, wgs=6), dict(kernel=1, op=1, seed=4),
               dict(nd=3, wait=3, span=1, op=0, seed=5, first_piece=1)):
        rc, f, err = run(model["tsan"], tiles=150, launches=2, timeout=300, **kw)
        assert "ThreadSanitizer" not in err, (kw, err[-3000:])
        assert rc == 0 and f["ok"] == "1", (kw, f)


def test_thread_sanitizer_sees_a_ring_reused_too_early(model):
    """The check can fail: with a ring far too short (3 slots for WAIT = 3) slots are
    rewritten while other waves still read them, which ThreadSanitizer reports."""
    if model["tsan"] is None:
        pytest.skip("ThreadSanitizer build not available")
    rc, f, err = run(model["tsan"], wait=3, slots=3, tiles=150, seed=1, spin=20000, timeout=300)
    assert "ThreadSanitizer: data race" in err
