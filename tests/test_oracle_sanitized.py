"""The oracle's pins, run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of the same C source.

The oracle does its own index arithmetic (neighbour offsets, block members,
summary strides) and allocates per-thread scratch, so an out-of-bounds read,
a leak-free use-after-free or signed overflow would not necessarily change a
result. Here the pin functions of the sensitivity suite run in a child
process whose oracle library is the sanitized build (with the sanitizer
runtimes preloaded); any report aborts the child with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PINS = ["pin_rope", "pin_rope_sequence", "pin_neighbours", "pin_local", "pin_summaries",
        "pin_global", "pin_mix", "pin_summary_centre", "pin_gqa", "pin_backward"]

CHILD = r"""
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle
import test_oracle_pin_sensitivity as ps
with oracle.use_library({lib!r}):
    for name in {pins!r}:
        assert getattr(ps, name)(), name
        print(name, "ok", flush=True)
"""


def _run_child(lib, preload, pins):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    # python itself is not instrumented: its allocations are not leaks of ours,
    # and the interpreter's own teardown is not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    code = CHILD.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=lib, pins=pins)
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=600)


@pytest.fixture(scope="module")
def sanitized_lib():
    from oracle import build as ob
    try:
        return ob.build_sanitized(), ob.sanitizer_preload()
    except (subprocess.CalledProcessError, FileNotFoundError) as e:  # pragma: no cover
        pytest.skip(f"no sanitizer toolchain: {e}")


def test_pins_pass_under_asan_and_ubsan(sanitized_lib):
    lib, preload = sanitized_lib
    r = _run_child(lib, preload, PINS)
    assert r.returncode == 0, f"sanitized oracle failed:\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert r.stdout.count(" ok") == len(PINS)


def test_sanitizer_reports_a_planted_overflow(sanitized_lib, tmp_path):
    """The harness is live: an edge check off by one (a neighbour one site
    past the last plane reads past the slot map) is reported by ASan."""
    from oracle import build as ob
    _, preload = sanitized_lib
    src = open(ob.SRC).read()
    old = "z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])\n    return -1;"
    assert src.count(old) == 1
    path = tmp_path / "overflow.c"
    path.write_text(src.replace(old, old.replace("z >= d->grid[0]", "z > d->grid[0]")))
    so = tmp_path / "overflow_san.so"
    subprocess.run(["gcc", *ob.SAN_FLAGS, "-std=c11", "-fopenmp", "-shared", "-fPIC", str(path),
                    "-o", str(so), "-lm"], check=True)
    r = _run_child(str(so), preload, ["pin_neighbours"])
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr
