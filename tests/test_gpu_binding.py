"""The binding's fast path (2-D row-major tensors on the current device,
torch's current stream) against its general path: bit-identical results,
and the same errors for calls the fast path does not cover."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def glu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    from mlp_gated_activation_amd import glu as g
    return g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_fast_and_general_paths_agree(glu, dtype):
    g = torch.Generator(device="cuda").manual_seed(1)
    a = (2 * torch.randn(37, 1000, device="cuda", generator=g)).to(dtype)
    b = torch.randn(37, 1000, device="cuda", generator=g).to(dtype)
    dy = torch.randn(37, 1000, device="cuda", generator=g).to(dtype)
    for kind in ("silu", "gelu_erf", "gelu_tanh", "relu"):
        y2 = glu.glu_fwd(kind, "separate", a, b)                           # fast path
        y3 = glu.glu_fwd(kind, "separate", a.view(1, 37, 1000), b.view(1, 37, 1000))   # general path
        assert torch.equal(y2, y3.view(37, 1000))
        yi = glu.glu_fwd(kind, "separate", a, b.clone(), inplace=True)
        assert torch.equal(yi, y2)
        a2, b2 = a.clone(), b.clone()
        glu.glu_bwd(kind, "separate", a2, b2, dy, inplace=True)            # fast path
        a3, b3 = a.clone().view(1, 37, 1000), b.clone().view(1, 37, 1000)
        glu.glu_bwd(kind, "separate", a3, b3, dy.view(1, 37, 1000), inplace=True)
        assert torch.equal(a2, a3.view(37, 1000)) and torch.equal(b2, b3.view(37, 1000))
    # padded rows (row stride > cols) take the fast path too
    ap = torch.zeros(37, 1024, device="cuda", dtype=dtype)[:, :1000]
    ap.copy_(a)
    assert torch.equal(glu.glu_fwd("silu", "separate", ap, b), glu.glu_fwd("silu", "separate", a, b))


def test_errors_match_the_general_path(glu):
    a = torch.randn(8, 64, device="cuda").to(torch.bfloat16)
    b = torch.randn(8, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        glu.glu_fwd("silu", "separate", a, b.half())
    with pytest.raises(ValueError, match="shape"):
        glu.glu_fwd("silu", "separate", a, b[:, :32])
    with pytest.raises(ValueError, match="contiguous"):
        glu.glu_fwd("silu", "separate", a, b, y=torch.empty(64, 8, device="cuda", dtype=torch.bfloat16).t())
    with pytest.raises(ValueError, match="inplace"):
        glu.glu_fwd("silu", "separate", a, b, y=torch.empty_like(a), inplace=True)
    with pytest.raises(ValueError, match="unknown kind"):
        glu.glu_fwd("swish", "separate", a, b)
    buf = torch.empty(8 * 64 + 1, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(glu.GluError, match="GLU_ERR_ALIAS"):     # y over a, one element off
        glu.glu_fwd("silu", "separate", buf[:512].view(8, 64), b, y=buf[1:513].view(8, 64))
    with pytest.raises(ValueError, match="ROCm"):
        glu.glu_fwd("silu", "separate", a.cpu(), b.cpu())
    with pytest.raises(ValueError):
        glu.glu_bwd("silu", "separate", a, b, torch.randn(8, 32, device="cuda").to(torch.bfloat16))
