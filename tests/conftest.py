import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# ORACLE_MUTATION=<n>: plant slip n of oracle_mutations.MUTATIONS in the oracle for
# this run (used by test_oracle_mutations.py, which expects the pins to fail).
if os.environ.get("ORACLE_MUTATION"):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle_mutations
    oracle_mutations.install(int(os.environ["ORACLE_MUTATION"]))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
