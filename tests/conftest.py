import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C-ABI")


def pytest_sessionstart(session):
    # build the HIP library in-tree when it is missing (never rebuilds)
    lib = os.path.join(ROOT, "paged_decode_attention_splitk_amd", "libpda.so")
    if not os.path.exists(lib):
        import importlib.util
        path = os.path.join(ROOT, "paged_decode_attention_splitk_amd", "_build.py")
        spec = importlib.util.spec_from_file_location("pda_build", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)   # by path: never loads a stale library first
        mod.build(verbose=True)
