"""Every slip of oracle_mutations.MUTATIONS, planted alone, makes at least one CPU
pin fail: the pins of test_oracle_pins.py and test_oracle_quant_pins.py are run
in a child process with the slip planted (and once without, which must pass)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutations import MUTATIONS

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = [os.path.join(HERE, "test_oracle_pins.py"), os.path.join(HERE, "test_oracle_quant_pins.py")]


def _run_pins(index=None):
    env = dict(os.environ, OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2", MKL_NUM_THREADS="2")
    env.pop("ORACLE_MUTATION", None)
    if index is not None:
        env["ORACLE_MUTATION"] = str(index)
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=os.path.dirname(HERE), env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    return p.returncode, p.stdout


@pytest.mark.skipif(bool(os.environ.get("ORACLE_MUTATION")), reason="already inside a planted run")
def test_every_planted_slip_fails_a_pin():
    rc, out = _run_pins()
    assert rc == 0, "the pins must pass on the unchanged oracle:\n" + out[-2000:]
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_pins, range(len(MUTATIONS))))
    survivors = []
    for (name, *_), (rc, out) in zip(MUTATIONS, results):
        if rc == 0:
            survivors.append(name)
        else:
            # the child must have failed a pin, not crashed on the planting itself
            assert "failed" in out, f"slip {name!r}: pins did not run:\n{out[-2000:]}"
    assert not survivors, f"slips that pass every pin: {survivors}"
