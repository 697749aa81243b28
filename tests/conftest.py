import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle, built with gcc only if no build is present.

    KVBT_ORACLE_LIB names another build of it (a planted-mistake variant)."""
    import oracle
    mutant = os.environ.get("KVBT_ORACLE_LIB")
    if mutant:       # set only by the mutation test, which plants a mistake on purpose
        return oracle.Oracle(mutant)
    oracle.build(force=False)
    return oracle.default()


@pytest.fixture(scope="session")
def attn_oracle():
    """The sparse-attention oracle module (oracle/sparse_attn.py).

    KVBT_ATTN_ORACLE_SRC names another copy of its source (a planted-mistake variant)."""
    src = os.environ.get("KVBT_ATTN_ORACLE_SRC")
    if src:          # set only by the mutation test, which plants a mistake on purpose
        import importlib.util
        spec = importlib.util.spec_from_file_location("sparse_attn_variant", src)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod
    from oracle import sparse_attn
    return sparse_attn


@pytest.fixture(scope="session")
def index_oracle():
    """The index-score oracle module (oracle/index_scores.py).

    KVBT_INDEX_ORACLE_SRC names another copy of its source (a planted-mistake variant)."""
    src = os.environ.get("KVBT_INDEX_ORACLE_SRC")
    if src:          # set only by the mutation test, which plants a mistake on purpose
        import importlib.util
        spec = importlib.util.spec_from_file_location("index_scores_variant", src)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod
    from oracle import index_scores
    return index_scores
