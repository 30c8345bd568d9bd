import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    import oracle
    oracle.build(force=False)
    yield


_NAMED = {}


@pytest.fixture(scope="session")
def named_reference():
    """The five named workloads and the oracle's full result on each, every
    (node, head) row, computed once per session: ``get(name) -> (w, out,
    lse)``.  The largest (32 requests of 256 nodes over 4096-token
    prefixes) is about 550 GFLOP of fp64 work, tens of seconds on the
    oracle's thread pool, so it is shared between the test files."""
    import oracle
    from tree_masked_attention_plan_amd import workloads as W

    def get(name):
        if name not in _NAMED:
            w = W.make_config(name)
            print(f"[oracle] full reference for {name}: N={w.N} rows={w.N * w.Hq}", flush=True)
            o, l = oracle.tree_attn_workload(w)
            _NAMED[name] = (w, o, l)
        return _NAMED[name]

    yield get
    _NAMED.clear()
