import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# GPU test modules of the rows beyond the hot path itself (the key-split
# streaming call, guidance, grouped heads, the rest of the layer, the
# shifted-schedule sampler loop) run after the hot path's own: under -x a
# failure there must not hide the hot path's results.
LATER = ("test_gpu_split.py", "test_gpu_cfg_gqa.py", "test_gpu_block.py", "test_gpu_sampler.py")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(session, config, items):
    items.sort(key=lambda it: os.path.basename(str(it.fspath)) in LATER)
