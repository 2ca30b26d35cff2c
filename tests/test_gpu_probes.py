"""The reference probes the measurements are stated against.  The
matrix-core rate probe computes what it claims: with every operand 1.0 each
lane's sum of its 256 accumulator values is exactly 256 x 16 (bf16,
32x32x16) or 256 x 64 (E4M3, 32x32x64) per round, and with hashed operands
two calls give the same finite sums."""
import pytest
import torch

from combine_router_top_expert_amd import mok_mfma_probe
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
