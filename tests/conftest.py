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
        from paged_kv_decode_12_amd import build as _b
        _b.build(force=True)
