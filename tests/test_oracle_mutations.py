"""Every planted mistake in the CPU oracle fails at least one of its pins.

Runs tests/test_oracle_pins.py in child processes, once with the oracle as
it is (it must pass) and once per mutation of tests/oracle_mutations.py (each
run must end with failed tests, not with an error of the harness).  The
mutations are plausible mistakes in writing the oracle from the pages: a
wrong chunk rule, a lost row, alignment ignored, rounding half up or by
truncation, padding left unset, every piece read from row 0, a rank's
contribution dropped, no division by N or a multiply by a rounded 1/N (bf16
and fp32 contributions), each AdamW term dropped or swapped,
the update's sign flipped, eps inside the square root, optimizer state not
sharded in the accounting (optimizer state, gradients), FP8 overflow to
NaN or ties away from zero, resharding offsets taken from the wrong side or
the last source rank skipped, NaNs rounded like numbers in the bf16 cast,
accumulation restarted by adding to +0, the reduce-scatter rows reversed,
the second moment without the square, amax of signed values, the FP8
scale divided, e4m3 decoded with bias 8, pieces in reverse registration
order, decay without the learning rate, pieces starting a row late.  CPU
only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from oracle_mutations import MUTATIONS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")


def _run(name):
    env = dict(os.environ)
    env.pop("FSDP_ORACLE_MUTATION", None)
    if name is not None:
        env["FSDP_ORACLE_MUTATION"] = name
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, (r.stdout + r.stderr)[-1500:]


def test_every_planted_mistake_fails_a_pin():
    names = [None] + sorted(MUTATIONS)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        results = {n: (rc, out) for n, rc, out in ex.map(_run, names)}
    rc, out = results.pop(None)
    assert rc == 0, "the pins fail on the oracle itself:\n" + out
    # pytest's exit code 1: tests ran and some failed; anything else is the
    # harness, not a pin, stopping the run
    survived = {n: (rc, out) for n, (rc, out) in results.items() if rc != 1}
    assert not survived, "\n".join(f"{n}: exit {rc}\n{out}" for n, (rc, out) in survived.items())
