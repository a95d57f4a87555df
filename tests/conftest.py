import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Host sanitizer runs (CPU only): RAC_SANITIZED=1 loads the ASan/UBSan builds
    # of the C ABI's host code and of the oracle from _build/asan (built by
    # `python -m rotary_position_embedding_causal_amd.build --sanitize` and
    # `python -m oracle.build --sanitize`); the ROCm clang's ASan runtime must
    # be preloaded into the interpreter (LD_PRELOAD).
    if os.environ.get("RAC_SANITIZED") == "1":
        import oracle
        import rotary_position_embedding_causal_amd as rac
        rac.LIB_PATH = os.path.join(ROOT, "_build", "asan", "librac.so")
        oracle.LIB_PATH = os.path.join(ROOT, "_build", "asan", "liboracle.so")
        os.environ["ORACLE_SANITIZE"] = "1"  # the mutant copies too


@pytest.fixture(scope="session")
def orc():
    """The fp64 CPU oracle (built from oracle/rac_oracle.c if no build exists)."""
    import oracle
    return oracle.default()
