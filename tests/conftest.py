import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# tests/test_oracle_mutations.py runs the oracle's pins in child processes
# with one planted mistake each, named by this variable; it is never set in
# an ordinary run
_MUTATION = os.environ.get("FSDP_ORACLE_MUTATION")
if _MUTATION:
    import oracle_mutations

    oracle_mutations.apply(_MUTATION)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Non-comment, non-empty lines of a golden fixture."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#", 1)[0].strip() for ln in f
                if ln.split("#", 1)[0].strip()]


def golden_kv(name):
    out = {}
    for ln in read_golden(name):
        if ":" in ln:
            k, v = ln.split(":", 1)
            out[k.strip()] = v.split()
    return out


def parse_shape(tok):
    return tuple(int(x) for x in tok.split("x"))


@pytest.fixture(scope="session")
def golden():
    return read_golden, golden_kv
