"""The library's measurement copy kernel (colibri_moe_stream_copy): a byte
exact copy, also for sizes that leave a ragged tail after its unrolled
grid-stride loop."""
import pytest

import sparse_moe_gemm_amd as cm

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1000003, 64 << 20])
def test_stream_copy_is_exact(nbytes):
    import torch

    g = torch.Generator(device="cpu").manual_seed(nbytes % 1009)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    print(f"stream_copy {nbytes} bytes", flush=True)
    cm.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
