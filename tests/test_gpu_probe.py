"""The matrix-unit peak probe (moe_probe_mfma) on the GPU: the flop count it
reports and the checksum it writes.  The loop multiplies constant operands
into four accumulators, so every lane's checksum is a finite sum that an
independent fp64 computation of the same products bounds."""
import numpy as np
import pytest
import torch

import sparsely_gated_mixture_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,per_instr", [(moe.MOE_BF16, 32768), (moe.MOE_F32, 4096)])
def test_probe_flops_and_checksum(dtype, per_instr):
    blocks, iters = 16, 10
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = moe.moe_probe_mfma(dtype, blocks, iters, sink)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 4 * per_instr
    s = sink.cpu().numpy()
    assert np.isfinite(s).all()
    # Operands are at most 0.007 and 0.014; each accumulator element sums
    # iters * K products (K = 16 or 2), 4 accumulators x 16 elements per lane.
    K = 16 if dtype == moe.MOE_BF16 else 2
    bound = 4 * 16 * iters * K * 0.014 * 0.014
    assert np.all(np.abs(s) <= bound * 1.01)
    assert np.any(s != 0)


def test_hbm_read_probe_reads_every_chunk():
    # Block b reads chunks [b*per, min(n16, (b+1)*per)), per = ceil(n16 /
    # blocks); thread t's checksum is the xor over the chunks of its block's
    # segment at offsets t modulo 256, folded to its low 16 bits.
    blocks = 4
    n16 = blocks * 256 * 8 * 3 + 77  # several 32 KB rounds per block and a ragged tail
    g = torch.Generator().manual_seed(5)
    words = torch.randint(0, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int64)
    buf = words.to(torch.int32).cuda()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    moe.moe_probe_hbm_read(buf, n16 * 16, blocks, sink)
    torch.cuda.synchronize()
    w = words.numpy().astype(np.uint32).reshape(n16, 4)
    chunk = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    per = -(-n16 // blocks)
    expect = np.zeros(blocks * 256, np.uint32)
    for b in range(blocks):
        seg = chunk[b * per:min(n16, (b + 1) * per)]
        for t in range(256):
            expect[b * 256 + t] = np.bitwise_xor.reduce(seg[t::256]) if t < len(seg) else 0
    np.testing.assert_array_equal(sink.cpu().numpy(), (expect & 0xFFFF).astype(np.float32))
