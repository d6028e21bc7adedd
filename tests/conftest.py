import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# GPU parity files in the order they run: the index-selected decode path first, then
# the matrix-core shapes, latent attention, graph capture, and the rows beyond the
# attention ops. Files not listed run after these, in their usual order.
GPU_ORDER = ("test_gpu_qsa.py", "test_gpu_mfma.py", "test_gpu_latent.py", "test_gpu_graph.py",
             "test_gpu_dense.py", "test_gpu_compress.py", "test_gpu_select.py", "test_gpu_scale.py",
             "test_gpu_batches.py", "test_gpu_shapes.py")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(session, config, items):
    def rank(item):
        name = os.path.basename(str(item.fspath))
        if name.startswith("test_zz"):
            return len(GPU_ORDER) + 1          # collected last on purpose
        return GPU_ORDER.index(name) if name in GPU_ORDER else -1
    # stable: CPU-only files keep their order in front, GPU files follow GPU_ORDER
    items[:] = sorted(items, key=rank)
