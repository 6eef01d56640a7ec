import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Mutation testing of the oracle (tests/test_oracle_mutations.py): a child
# pytest process gets a planted-mistake copy of one oracle module (named by
# GSA_ORACLE_MUTANT_MODULE, default gsa_oracle) through this variable and must
# then fail its pins.  Never set in ordinary runs.
_MUTANT = os.environ.get("GSA_ORACLE_MUTANT")
if _MUTANT:
    import oracle  # noqa: E402  (the package; the module is replaced below)
    _name = os.environ.get("GSA_ORACLE_MUTANT_MODULE", "gsa_oracle")
    _spec = importlib.util.spec_from_file_location("oracle." + _name, _MUTANT)
    _mod = importlib.util.module_from_spec(_spec)
    sys.modules["oracle." + _name] = _mod
    _spec.loader.exec_module(_mod)
    setattr(oracle, _name, _mod)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
