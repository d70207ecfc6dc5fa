"""The HBM bandwidth probes behind bench.py --ceiling: the copy copies every
byte, the read leaves its sink alone (its fold of the data never equals the
marker value for this input)."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_copy_and_read():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as svla
    lib = svla.library()
    n, wgs = 32 << 20, 64
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros_like(src)
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda:0")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.svla_hbm_probe(1, p(src), p(dst), n, None, wgs, st) == 0
    assert lib.svla_hbm_probe(0, p(src), None, n, p(sink), wgs, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert torch.count_nonzero(sink).item() == 0
