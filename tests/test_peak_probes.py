"""The achievable-peak probes (libssd_probe.so) that bench.py quotes its roofline
fractions against: the library exports its entry points and rejects bad
arguments on the host (no GPU), the copy copies and the MFMA loop computes its
closed form (GPU)."""
import ctypes

import pytest

from mamba2_ssd_chunked_amd import probes


def test_probe_library_exports_and_rejects_bad_arguments():
    lib = probes.load()
    for n in probes.SYMBOLS:
        assert hasattr(lib, n), n
    # rejected on the host, before any launch
    assert lib.ssd_probe_copy(None, None, 1024, None) == -1
    assert lib.ssd_probe_copy(ctypes.c_void_p(16), ctypes.c_void_p(32), 1000, None) == -1
    # a workgroup moves 4 KiB: sizes that are not whole workgroups are refused
    assert lib.ssd_probe_copy(ctypes.c_void_p(16), ctypes.c_void_p(32), 1024, None) == -1
    assert lib.ssd_probe_copy(ctypes.c_void_p(16), ctypes.c_void_p(32), 4096 + 2048, None) == -1
    assert lib.ssd_probe_copy(ctypes.c_void_p(8), ctypes.c_void_p(32), 1024, None) == -1
    assert lib.ssd_probe_mfma(None, 1, 1, 16, None) == -1
    assert lib.ssd_probe_mfma(ctypes.c_void_p(16), 0, 1, 16, None) == -1
    assert lib.ssd_probe_mfma(ctypes.c_void_p(16), 1, 0, 16, None) == -1
    assert lib.ssd_probe_mfma(ctypes.c_void_p(16), 1, 1, 8, None) == -1
    # 2048 workgroups x 4 waves x 10 rounds x (8 chains x 16*16*32*2 | 4 chains x 32*32*16*2)
    assert lib.ssd_probe_mfma_flops(2048, 10, 16) == 2048 * 4 * 10 * 8 * 16384
    assert lib.ssd_probe_mfma_flops(2048, 10, 32) == 2048 * 4 * 10 * 4 * 32768


@pytest.mark.gpu
def test_copy_probe_copies_and_stays_in_bounds():
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(7)
    n = (3 << 20) // 4
    guard = 1 << 16  # int32 words on either side of both buffers
    src_all = torch.randint(-2**31, 2**31 - 1, (n + 2 * guard,), generator=g,
                            dtype=torch.int32).to(dev)
    dst_all = torch.full((n + 2 * guard,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    before = dst_all.clone()
    probes.probe_copy(src_all[guard:guard + n], dst_all[guard:guard + n])
    torch.cuda.synchronize()
    assert torch.equal(src_all[guard:guard + n], dst_all[guard:guard + n])
    # nothing written outside the destination
    assert torch.equal(dst_all[:guard], before[:guard])
    assert torch.equal(dst_all[guard + n:], before[guard + n:])


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [16, 32])
def test_mfma_probe_closed_form(shape):
    import torch
    out = torch.full((8 * 256,), -1.0, dtype=torch.float32, device="cuda:0")
    flops = probes.probe_mfma(out, 8, 100, shape)
    torch.cuda.synchronize()
    # chain c's elements are c + 100 rounds x K products of (1/64)^2
    want = (4 * (0 + 1 + 2 + 3 + 4 + 5 + 6 + 7) + 8 * 4 * 100 * 32 / 4096 if shape == 16
            else 16 * (0 + 1 + 2 + 3) + 4 * 16 * 100 * 16 / 4096)
    assert probes.mfma_expected(100, shape) == want
    assert torch.all(out == want)
    assert flops == 8 * 4 * 100 * (8 * 16384 if shape == 16 else 4 * 32768)
