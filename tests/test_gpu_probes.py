"""GPU checks of the measurement probes (not the MTTKRP): the read probe
touches every byte of its buffer exactly once (its per-workgroup checksums add
up to the buffer's), and the MFMA probe writes finite values.  Through the
C ABI."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mttkrp_matrix_free_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nwords", [4, 4 * 1000003, 4 * (1 << 22)])
def test_read_probe_reads_every_byte(nwords):
    L = _lib.lib()
    g = torch.Generator().manual_seed(nwords)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nwords,), dtype=torch.int64, generator=g)
    host = host.to(torch.int32)
    buf = host.cuda()
    sink = torch.zeros(L.mttkrp_probe_read_grid(), dtype=torch.int32, device="cuda")
    st = L.mttkrp_probe_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nwords * 4),
                             ctypes.c_void_p(sink.data_ptr()), None)
    assert st == 0
    torch.cuda.synchronize()
    w = host.numpy().view(np.uint32).reshape(-1, 4)
    per_group = (w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]).astype(np.uint64)
    expect = int(per_group.sum() % (1 << 32))
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    assert got == expect


def test_read_probe_rejects_bad_arguments():
    L = _lib.lib()
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(L.mttkrp_probe_read_grid(), dtype=torch.int32, device="cuda")
    assert L.mttkrp_probe_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(20),
                               ctypes.c_void_p(sink.data_ptr()), None) == _lib.EINVAL
    assert L.mttkrp_probe_read(ctypes.c_void_p(buf.data_ptr() + 4), ctypes.c_size_t(16),
                               ctypes.c_void_p(sink.data_ptr()), None) == _lib.EALIGN


@pytest.mark.parametrize("eb", [8, 4])
def test_mfma_probe_finite(eb):
    L = _lib.lib()
    sink = torch.full((4 * L.mttkrp_probe_mfma_grid(),), float("nan"), dtype=torch.float64,
                      device="cuda")
    assert L.mttkrp_probe_mfma(eb, ctypes.c_int64(64), ctypes.c_void_p(sink.data_ptr()), None) == 0
    torch.cuda.synchronize()
    v = sink.cpu().numpy()
    assert np.all(np.isfinite(v)) and np.all(v > 0)
    assert L.mttkrp_probe_mfma(2, ctypes.c_int64(64), ctypes.c_void_p(sink.data_ptr()), None) \
        == _lib.EINVAL
