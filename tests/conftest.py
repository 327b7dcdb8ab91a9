import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # build what is missing (never rebuilds an existing library)
    import oracle
    oracle.build(force=False)
    lib = os.path.join(ROOT, "paged_kv_decode_12_amd", "libpkvd.so")
    if not os.path.exists(lib):
        _build_module().build(force=True)


def _build_module():
    """The package's build script, loaded by path (importing the package loads
    libpkvd.so, which is what is missing here)."""
    import importlib.util
    path = os.path.join(ROOT, "paged_kv_decode_12_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_pkvd_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod
