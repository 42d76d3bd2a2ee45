"""The measured-ceiling diagnostic (kvs_measure_peaks) through the C ABI:
it runs, returns plausible rates for an MI355X (a dense bf16 MFMA loop and a
streaming HBM read; published peaks 2.5 PFLOP/s and 8 TB/s), and rejects a
buffer that is too small on the host."""

import ctypes

import pytest
import torch

import kv_cache_eviction_amd as kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda:0")


def test_measured_peaks_plausible(dev):
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    tf, gb = kv.kvs_measure_peaks(buf)
    print("measured: %.1f TFLOP/s bf16 MFMA, %.1f GB/s HBM read" % (tf, gb))
    # loose bounds: a box far below these is broken, none can exceed the spec by much
    assert 1000.0 < tf < 2.6 * 1000.0
    assert 2000.0 < gb < 8.4 * 1000.0


def test_small_buffer_rejected(dev):
    lib = kv.load()
    tf, gb = ctypes.c_float(), ctypes.c_float()
    rc = lib.kvs_measure_peaks(ctypes.c_void_p(0x1000), 1 << 20, ctypes.byref(tf), ctypes.byref(gb),
                               None)
    assert rc == 1 and "66 MiB" in kv.last_error()
