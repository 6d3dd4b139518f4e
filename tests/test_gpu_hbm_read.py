"""moe_hbm_read (the plain-read floor the benchmark sets the expert FFN against) launches over
ragged sizes, from offsets inside a buffer, and leaves the buffer unchanged."""
import pytest
import torch

import moe_expert_offload_amd as M

pytestmark = pytest.mark.gpu


def test_hbm_read_ragged_sizes_leave_the_buffer_unchanged():
    buf = torch.randint(0, 256, (8 << 20,), dtype=torch.uint8, device="cuda")
    ref = buf.clone()
    # one word; part of one workgroup's span; several spans plus a tail; an exact multiple of the span
    for off, n in [(0, 16), (256, 16 * 1000), (4096, (3 << 20) + 48), (0, 8 << 20)]:
        print("hbm_read offset", off, "bytes", n, flush=True)
        M.hbm_read(buf, off, n)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


def test_hbm_read_python_range_check():
    buf = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MoeError):
        M.hbm_read(buf, 16, 4096)
    with pytest.raises(M.MoeError):
        M.hbm_read(buf, 8, 16)  # unaligned
