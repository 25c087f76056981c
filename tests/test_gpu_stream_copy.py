"""kda_stream_copy (the bandwidth measuring stick): a bit-exact copy at sizes that end inside a
wave's piece, a workgroup's round and the grid's stride, called through the C ABI."""

import ctypes

import pytest
import torch

import gated_delta_rule_67_amd as kda
from tests.helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 * (1 << 20) + 48, 64 << 20, (64 << 20) * 3 + 16 * 257])
def test_stream_copy_is_exact(nbytes):
    log(f"stream copy {nbytes} bytes")
    gen = torch.Generator().manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")  # 64 guard bytes after
    rc = kda.library().kda_stream_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                       nbytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == kda.KDA_OK, kda.status_string(rc)
    assert torch.equal(dst[:nbytes], src)
    assert torch.count_nonzero(dst[nbytes:]) == 0


def test_stream_copy_binding():
    src = torch.randn(1 << 20, device="cuda")
    dst = torch.empty_like(src)
    kda.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
