import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (large workloads)")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    """Write the test id to the real stderr before a GPU test runs, so a run
    that dies inside a kernel still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-test] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


def poison_(t):
    """Fill a device buffer with a value no kernel writes: NaN for floating
    tensors (bf16 0x7FC0, fp32 0x7FC00000), 0xFF bytes otherwise (a NaN in
    every float32 or bf16 view of a byte workspace)."""
    if t.is_floating_point():
        t.fill_(float("nan"))
    else:
        t.fill_(-1 if t.is_signed() else (1 << (8 * t.element_size())) - 1)
    return t


@pytest.fixture(autouse=True)
def _poison_library_buffers(request, monkeypatch):
    """In GPU tests, every buffer the binding allocates (outputs, the
    attention output and statistics of the training forward, gradients,
    workspaces, streaming state) starts as NaN or 0xFF bytes instead of
    whatever the caching allocator hands back, so a row, cell or flag a
    kernel leaves unwritten shows up as a NaN rather than as a stale value
    that may already be right."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch
    from chunked_attention_memory_amd import gecko

    original = gecko._empty

    def poisoned_empty(shape, dtype, device, stream):
        t = original(shape, dtype, device, stream)
        if stream is None:
            return poison_(t)
        with torch.cuda.stream(stream):
            return poison_(t)

    monkeypatch.setattr(gecko, "_empty", poisoned_empty)
    yield
