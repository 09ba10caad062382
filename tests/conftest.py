import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def _ensure_built():
    # load what is built; build only what is missing (hipcc cross-compiles here)
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "libk3oracle.so")):
        oracle.build()
    so = os.path.join(ROOT, "mxfp4_routed_expert_softmax_amd", "libk3moe.so")
    if not os.path.exists(so):
        from mxfp4_routed_expert_softmax_amd import build as b
        b.build()


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
