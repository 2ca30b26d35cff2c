"""The reference probes the measurements are stated against.  The
matrix-core rate probe computes what it claims: with every operand 1.0 each
lane's sum of its 256 accumulator values is exactly 256 x 16 (bf16,
32x32x16) or 256 x 64 (E4M3, 32x32x64) per round, and with hashed operands
two calls give the same finite sums.  The HBM streaming probe moves the
bytes it claims: its copy is the source, its write fills every word, and
its read leaves the destination alone."""
import pytest
import torch

from combine_router_top_expert_amd import mok_hbm_stream, mok_mfma_probe
from test_gpu_parity import DEV, _log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,k_per_mfma", [(0, 16), (1, 64)])
def test_mfma_probe_sums(kind, k_per_mfma):
    _log(f"mfma probe kind {kind}")
    wgs, iters = 8, 7
    out = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device=DEV)
    mok_mfma_probe(kind, 1, iters, wgs, out)
    torch.cuda.synchronize()
    assert torch.all(out == 256.0 * k_per_mfma * iters)
    a = torch.full_like(out, float("nan"))
    b = torch.full_like(out, float("nan"))
    mok_mfma_probe(kind, 0, iters, wgs, a)
    mok_mfma_probe(kind, 0, iters, wgs, b)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(a)) and torch.equal(a, b)


def test_hbm_stream_moves_its_bytes():
    _log("hbm stream probe")
    n = (3 << 20) + 4096 + 16                      # not a multiple of the 32 KiB chunk
    g = torch.Generator().manual_seed(20260)
    src = torch.randint(0, 1 << 30, (n // 4,), dtype=torch.int32, generator=g).to(DEV)
    dst = torch.zeros_like(src)
    mok_hbm_stream(2, dst, src, n)                 # copy
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    dst.zero_()
    mok_hbm_stream(1, dst, src, n)                 # write: the fill pattern everywhere
    torch.cuda.synchronize()
    assert torch.all(dst == 0x3F803F80)
    dst.zero_()
    mok_hbm_stream(0, dst, src, n)                 # read: the fold never equals the pattern here
    torch.cuda.synchronize()
    assert torch.all(dst == 0)
