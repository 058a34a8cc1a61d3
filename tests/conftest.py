import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases (minutes)")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    oracle.build(force=False)
    yield


def _lib_stale():
    pkg = os.path.join(ROOT, "paged_kv_cache_gqa_amd")
    lib = os.path.join(pkg, "libpagedattn.so")
    if not os.path.exists(lib):
        return True
    srcs = [os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))]
    srcs.append(os.path.join(ROOT, "include", "pagedattn.h"))
    return max(os.path.getmtime(s) for s in srcs) > os.path.getmtime(lib)


def load_builder():
    """The package's build script, loaded without importing the package
    (whose import loads the library)."""
    import importlib.util
    path = os.path.join(ROOT, "paged_kv_cache_gqa_amd", "build.py")
    spec = importlib.util.spec_from_file_location("paged_kv_cache_gqa_amd_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="session")
def palib():
    """The product library's Python binding (built first if missing or stale)."""
    if _lib_stale():
        load_builder().build()
    import paged_kv_cache_gqa_amd as pa
    return pa
