"""The oracle's pins catch plausible mistakes: each entry of ``oracle_mutants.MUTANTS`` rewrites one
statement of one oracle function (erase before decay, a dropped write, readout before the update,
swapped RDA gates, an off-by-one chunk ratio, a dropped gradient term, an off-by-one snapshot, a
rescaled activation, ...), and the pin file of that function's own module, run in a child process
with the mistake planted, must fail (the step rule and the chunked form by the closed forms and
hand-worked examples of ``test_oracle_pins.py``, not only through the backward's finite
differences). A control run of every pin file with the plugin loaded and nothing planted must
pass. CPU only."""
import concurrent.futures as cf
import os
import subprocess
import sys

import oracle_mutants

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
PINS = sorted(os.path.join("tests", f) for f in os.listdir(TESTS) if f.startswith("test_oracle_")
              and f.endswith(".py") and f != "test_oracle_mutants.py")
# the pin file of each oracle module
OWN_PINS = {"recurrence": "test_oracle_pins.py", "chunked": "test_oracle_pins.py", "backward": "test_oracle_backward.py",
            "states": "test_oracle_states.py", "product": "test_oracle_product.py", "prep": "test_oracle_prep.py"}


def _run_pins(mutant):
    files = [os.path.join("tests", OWN_PINS[oracle_mutants.MUTANTS[mutant][0]])] if mutant else PINS
    env = dict(os.environ, DR_ORACLE_MUTANT=mutant,
               PYTHONPATH=os.pathsep.join([TESTS, ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-p", "oracle_mutants", "-x", "-q", "-m", "not gpu", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    failed = [ln.split(" - ")[0] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
    return r.returncode, (failed[0] if failed else r.stdout[-1500:] + r.stderr[-1500:])


def test_pins_catch_every_planted_mistake():
    assert len(PINS) >= 5
    names = [""] + sorted(oracle_mutants.MUTANTS)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(names, ex.map(_run_pins, names)))
    rc, out = results.pop("")
    assert rc == 0, f"control run (nothing planted) did not pass:\n{out}"
    survivors = {n: out for n, (rc, out) in results.items() if rc != 1}  # 1: some pin failed
    for n, (rc_n, out_n) in sorted(results.items()):
        print(f"[planted] {n}: {f'caught by {out_n}' if rc_n == 1 else f'NOT caught (pytest exit {rc_n})'}", flush=True)
    assert not survivors, "\n\n".join(f"{n}:\n{o}" for n, o in survivors.items())
