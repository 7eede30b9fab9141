"""The matrix-instruction loop behind the benchmark's attainable rates (libmla_attainable, GPU):
both instruction kinds run at one and at two workgroups per compute unit and leave finite,
non-zero sums, and a larger iteration count takes longer (the loop is not removed)."""
import ctypes
import os

import numpy as np
import pytest

from _common import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_latent_kv_40_amd", "libmla_attainable.so")


@pytest.fixture(scope="module")
def loop():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    if not os.path.exists(LIB):
        pytest.fail("libmla_attainable.so is not built (run __graft_entry__.build())")
    fn = ctypes.CDLL(LIB).mla_attainable_mfma_loop
    fn.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    return fn


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("per_cu", [1, 2])
def test_loop_runs_and_scales_with_iterations(loop, kind, per_cu):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * per_cu
    out = torch.zeros(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for iters in (64, 64, 1024):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = loop(kind, wgs, iters, 163840 // per_cu, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        times.append(e0.elapsed_time(e1))
        v = out.cpu().numpy()
        assert np.all(np.isfinite(v)) and np.count_nonzero(v) > 0.9 * v.size, (kind, per_cu, iters)
    log(f"  kind {kind}, {per_cu} workgroup(s) per CU: {times[1]:.3f} ms at 64 iterations, {times[2]:.3f} ms at 1024")
    assert times[2] > 2.0 * times[1]


@pytest.mark.parametrize("kind", [0, 1])
def test_read_streams_every_word_once(kind):
    """mla_attainable_read (the read streams behind the benchmark's attainable read bandwidth):
    the threads' wrapping sums add up to the buffer's word sum mod 2^32, for two slice lengths
    (one chunk per workgroup, and enough to fill the LDS ring several times), and the longer
    read takes longer."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    fn = ctypes.CDLL(LIB).mla_attainable_read
    fn.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int32
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * (1 if kind == 1 else 4)
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cpu").manual_seed(7 + kind)
    times = []
    for per in (1, 1, 9):
        words = torch.randint(-2 ** 31, 2 ** 31, (wgs * per * 36864 // 4,), dtype=torch.int64, generator=g)
        buf = words.to(torch.int32).to("cuda")
        out = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
        log(f"  read kind {kind}: {wgs} workgroups x {per} chunks")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = fn(kind, buf.data_ptr(), buf.numel() * 4, wgs, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        times.append(e0.elapsed_time(e1))
        want = int(words.sum().item()) % (1 << 32)
        got = int(out.cpu().to(torch.int64).sum().item()) % (1 << 32)
        assert got == want, (kind, per, got, want)
    log(f"  read kind {kind}: {times[1]:.3f} ms at 1 chunk per workgroup, {times[2]:.3f} ms at 9")
    assert times[2] > times[1]
