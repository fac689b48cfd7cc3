"""GPU tests of the autograd functions and the gated-MLP module.

The activation and its gradient must match the fp64 oracle to one output
ulp (they are the C-ABI kernels); the whole MLP must match a float64 CPU
reference of the same network within bf16-GEMM error."""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.compare import compare

pytestmark = pytest.mark.gpu
FMT = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}
KINDS = ("silu", "gelu_erf", "gelu_tanh", "relu")


@pytest.fixture(scope="module")
def fn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conftest import ensure_built
    ensure_built()
    from mlp_gated_activation_amd import functional
    return functional


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def ok(got, ref, what):
    rep = compare(f64(got), ref, FMT[got.dtype])
    assert rep.ok, f"{what}: {rep}"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("inplace", [True, False])
def test_autograd_separate(fn, kind, inplace):
    g = torch.Generator().manual_seed(31)
    a0 = (torch.randn(300, 777, generator=g) * 2).to(torch.bfloat16).cuda().requires_grad_()
    b0 = torch.randn(300, 777, generator=g).to(torch.bfloat16).cuda().requires_grad_()
    dy = torch.randn(300, 777, generator=g).to(torch.bfloat16).cuda()
    fa, fb, fdy = f64(a0), f64(b0), f64(dy)
    # non-leaf inputs (as the outputs of the projections would be); x * 1 is exact
    a, b = a0 * 1, b0 * 1
    y = fn.gated_activation(a, b, kind, inplace_backward=inplace)
    ok(y, oracle.fwd(kind, fa, fb), f"{kind} y")
    y.backward(dy)
    rda, rdb = oracle.bwd(kind, fa, fb, fdy)
    ok(a0.grad, rda, f"{kind} da")
    ok(b0.grad, rdb, f"{kind} db")
    if not inplace:
        assert torch.equal(a.detach(), a0.detach()), "out-of-place backward modified a"


@pytest.mark.parametrize("kind", KINDS)
def test_autograd_fused(fn, kind):
    g = torch.Generator().manual_seed(37)
    x0 = (torch.randn(257, 2 * 1000, generator=g) * 1.5).to(torch.float16).cuda().requires_grad_()
    dy = torch.randn(257, 1000, generator=g).to(torch.float16).cuda()
    fx, fdy = f64(x0), f64(dy)
    y = fn.gated_activation(x0 * 1, None, kind)
    ok(y, oracle.fwd_gate_up(kind, fx), f"{kind} fused y")
    y.backward(dy)
    ok(x0.grad, oracle.bwd_gate_up(kind, fx, fdy), f"{kind} fused dx")


def test_leaf_inputs_out_of_place(fn):
    g = torch.Generator().manual_seed(41)
    a = (torch.randn(64, 512, generator=g) * 2).to(torch.bfloat16).cuda().requires_grad_()
    b = torch.randn(64, 512, generator=g).to(torch.bfloat16).cuda().requires_grad_()
    keep_a, keep_b = a.detach().clone(), b.detach().clone()
    y = fn.swiglu(a, b, inplace_backward=False)
    y.sum().backward()
    assert torch.equal(a.detach(), keep_a) and torch.equal(b.detach(), keep_b)
    rda, rdb = oracle.bwd("silu", f64(keep_a), f64(keep_b), np.ones((64, 512)))
    ok(a.grad, rda, "leaf da")
    ok(b.grad, rdb, "leaf db")


def test_expanded_incoming_gradient(fn):
    """A broadcast (stride-0) incoming gradient goes to the strided kernels as is."""
    g = torch.Generator().manual_seed(43)
    a0 = (torch.randn(16, 256, generator=g) * 2).to(torch.bfloat16).cuda().requires_grad_()
    b0 = torch.randn(16, 256, generator=g).to(torch.bfloat16).cuda().requires_grad_()
    y = fn.geglu(a0 * 1, b0 * 1, approximate="tanh")
    row = torch.randn(1, 256, generator=g).to(torch.bfloat16).cuda()
    y.backward(row.expand(16, 256))
    rda, rdb = oracle.bwd("gelu_tanh", f64(a0), f64(b0), np.broadcast_to(f64(row), (16, 256)))
    ok(a0.grad, rda, "expanded dy da")
    ok(b0.grad, rdb, "expanded dy db")


def _reference_mlp(x, wgu, wd, kind, fused, inter):
    """float64 CPU reference of the same network with torch's own activations."""
    x = x.detach().cpu().double().requires_grad_()
    wgu = [w.detach().cpu().double().requires_grad_() for w in wgu]
    wd = wd.detach().cpu().double().requires_grad_()
    if fused:
        h = x @ wgu[0].t()
        gate, up = h[:, :inter], h[:, inter:]
    else:
        gate, up = x @ wgu[0].t(), x @ wgu[1].t()
    act = {"silu": F.silu, "relu": F.relu,
           "gelu_erf": lambda v: F.gelu(v, approximate="none"),
           "gelu_tanh": lambda v: F.gelu(v, approximate="tanh")}[kind]
    out = (act(gate) * up) @ wd.t()
    return x, wgu, wd, out


def _rel(got, ref):
    got = got.detach().cpu().double()
    ref = ref.detach().double()
    return float((got - ref).norm() / ref.norm())


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fused", [True, False])
def test_gated_mlp_matches_fp64_reference(fn, kind, fused):
    torch.manual_seed(47)
    hidden, inter, tokens = 256, 1000, 150
    mlp = fn.GatedMLP(hidden, inter, kind=kind, fused_gate_up=fused, device="cuda", dtype=torch.bfloat16)
    x = torch.randn(tokens, hidden, device="cuda", dtype=torch.bfloat16).requires_grad_()
    out = mlp(x)
    dout = torch.randn_like(out)
    out.backward(dout)
    wgu = [mlp.gate_up_proj.weight] if fused else [mlp.gate_proj.weight, mlp.up_proj.weight]
    rx, rw, rd, rout = _reference_mlp(x, wgu, mlp.down_proj.weight, kind, fused, inter)
    rout.backward(dout.detach().cpu().double())
    # bf16 GEMM inputs/outputs: a few 2^-8 relative per element, far less in norm
    tol = 2e-2
    assert _rel(out, rout) < tol
    assert _rel(x.grad, rx.grad) < tol
    assert _rel(mlp.down_proj.weight.grad, rd.grad) < tol
    for w, r in zip(wgu, rw):
        assert _rel(w.grad, r.grad) < tol


@pytest.mark.parametrize("kind", KINDS)
def test_gated_mlp_fused_epilogue(fn, kind):
    """The module with the gate/up projection and activation in one kernel:
    output and every gradient against the float64 reference, and the same
    as the unfused module to bf16-GEMM accuracy."""
    torch.manual_seed(53)
    hidden, inter, tokens = 256, 1000, 300
    mlp = fn.GatedMLP(hidden, inter, kind=kind, fused_epilogue=True, device="cuda", dtype=torch.bfloat16)
    x = torch.randn(2, tokens // 2, hidden, device="cuda", dtype=torch.bfloat16).requires_grad_()
    out = mlp(x)
    dout = torch.randn_like(out)
    out.backward(dout)
    w = mlp.gate_up_proj.weight
    rx, rw, rd, rout = _reference_mlp(x.reshape(tokens, hidden), [w], mlp.down_proj.weight, kind, True, inter)
    rout.backward(dout.reshape(tokens, hidden).detach().cpu().double())
    tol = 2e-2
    assert _rel(out.reshape(tokens, hidden), rout) < tol
    assert _rel(x.grad.reshape(tokens, hidden), rx.grad) < tol
    assert _rel(mlp.down_proj.weight.grad, rd.grad) < tol
    assert _rel(w.grad, rw[0].grad) < tol


@pytest.mark.parametrize("kind", KINDS)
def test_gated_mlp_auto_epilogue(fn, kind):
    """The default fused_epilogue="auto": the fused gate/up kernel for at most
    256 tokens of bf16/fp16 whose few-token tiles fill at most one round of
    workgroups, the unfused path otherwise; both agree with the float64
    reference, in output and every gradient."""
    torch.manual_seed(59)
    hidden, inter = 256, 1000
    mlp = fn.GatedMLP(hidden, inter, kind=kind, device="cuda", dtype=torch.bfloat16)
    w = mlp.gate_up_proj.weight
    for tokens, fused in ((16, True), (129, True), (256, True), (257, False), (300, False)):
        x = torch.randn(tokens, hidden, device="cuda", dtype=torch.bfloat16).requires_grad_()
        assert mlp.uses_fused_epilogue(x) is fused, tokens
        for q in mlp.parameters():
            q.grad = None
        out = mlp(x)
        dout = torch.randn_like(out)
        out.backward(dout)
        rx, rw, rd, rout = _reference_mlp(x, [w], mlp.down_proj.weight, kind, True, inter)
        rout.backward(dout.detach().cpu().double())
        tol = 2e-2
        assert _rel(out, rout) < tol, tokens
        assert _rel(x.grad, rx.grad) < tol, tokens
        assert _rel(mlp.down_proj.weight.grad, rd.grad) < tol, tokens
        assert _rel(w.grad, rw[0].grad) < tol, tokens
    # not where the few-token tiles need more than one workgroup per compute unit
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    wide = fn.GatedMLP(hidden, 64 * ncu + 1, device="cuda", dtype=torch.bfloat16)
    assert not wide.uses_fused_epilogue(x[:16])
    assert fn.GatedMLP(hidden, 64 * ncu, device="cuda", dtype=torch.bfloat16).uses_fused_epilogue(x[:16])
    # not for fp32, nor for a row stride the kernel cannot take
    assert not fn.GatedMLP(hidden, inter, device="cuda").uses_fused_epilogue(torch.randn(16, hidden, device="cuda"))
    xs = torch.randn(16, hidden + 4, device="cuda", dtype=torch.bfloat16)[:, :hidden]
    assert not mlp.uses_fused_epilogue(xs)
    assert not fn.GatedMLP(hidden, inter, fused_epilogue=False, device="cuda",
                           dtype=torch.bfloat16).uses_fused_epilogue(x[:16])


def test_gate_up_activation_inference_saves_nothing(fn):
    """Without gradients the forward writes no pre-activations."""
    x = torch.randn(64, 128, device="cuda", dtype=torch.bfloat16)
    w = (torch.randn(2 * 96, 128, device="cuda") * 0.05).to(torch.bfloat16)
    with torch.no_grad():
        h = fn.gate_up_activation(x, w, "silu")
    ref = F.silu(x.double() @ w[:96].double().t()) * (x.double() @ w[96:].double().t())
    assert _rel(h, ref.cpu()) < 1e-2


def test_module_rejects_unknown_kind(fn):
    with pytest.raises(ValueError):
        fn.GatedMLP(8, 8, kind="swish")
    with pytest.raises(ValueError):
        fn.geglu(torch.zeros(1, 8, device="cuda"), torch.zeros(1, 8, device="cuda"), approximate="fast")


def _rel_gpu(got, ref):
    return _rel(got, ref.detach().cpu())


@pytest.mark.parametrize("act", ["silu", "gelu", "gelu_pytorch_tanh"])
@pytest.mark.parametrize("fused", [True, False])
def test_drop_in_for_hf_llama_mlp(fn, act, fused):
    """GatedMLP.from_config on a Hugging Face LlamaConfig, loaded with a
    LlamaMLP's state dict, against that LlamaMLP itself: fp32, (batch, seq,
    hidden) input, forward and every gradient.  Both sides run the same
    torch GEMMs; only the activation step differs (here fp64 arithmetic,
    one rounding), so they agree to fp32 rounding."""
    transformers = pytest.importorskip("transformers")
    from transformers.models.llama.modeling_llama import LlamaMLP
    torch.manual_seed(5)
    cfg = transformers.LlamaConfig(hidden_size=128, intermediate_size=344, hidden_act=act)
    ref = LlamaMLP(cfg).to("cuda", torch.float32)
    mlp = fn.GatedMLP.from_config(cfg, fused_gate_up=fused).to("cuda", torch.float32)
    mlp.load_state_dict(ref.state_dict())
    x = torch.randn(3, 37, 128, device="cuda")
    xr = x.clone().requires_grad_()
    xm = x.clone().requires_grad_()
    yr = ref(xr)
    ym = mlp(xm)
    dy = torch.randn_like(yr)
    yr.backward(dy)
    ym.backward(dy)
    assert _rel_gpu(ym, yr) < 1e-5
    assert _rel_gpu(xm.grad, xr.grad) < 1e-5
    assert _rel_gpu(mlp.down_proj.weight.grad, ref.down_proj.weight.grad) < 1e-5
    if fused:
        gw = mlp.gate_up_proj.weight.grad
        assert _rel_gpu(gw[:344], ref.gate_proj.weight.grad) < 1e-5
        assert _rel_gpu(gw[344:], ref.up_proj.weight.grad) < 1e-5
    else:
        assert _rel_gpu(mlp.gate_proj.weight.grad, ref.gate_proj.weight.grad) < 1e-5
        assert _rel_gpu(mlp.up_proj.weight.grad, ref.up_proj.weight.grad) < 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
def test_recompute_activation_matches_and_saves_memory(fn, kind, dtype):
    """GatedMLP(recompute_activation=True) keeps only [gate | up] and
    recomputes act(gate) * up in the backward: the same output and gradients
    as the default module with the same weights (both run the same kernels
    and torch GEMMs), and a step's peak memory lower by about one
    tokens x intermediate activation."""
    torch.manual_seed(3)
    tokens, hidden, inter = 1024, 256, 2048
    base = fn.GatedMLP(hidden, inter, kind=kind, device="cuda", dtype=dtype)
    rec = fn.GatedMLP(hidden, inter, kind=kind, recompute_activation=True, device="cuda", dtype=dtype)
    rec.load_state_dict(base.state_dict())
    x = torch.randn(2, tokens // 2, hidden, device="cuda", dtype=dtype)
    dy = torch.randn(2, tokens // 2, hidden, device="cuda", dtype=dtype)

    def step(m):
        for q in m.parameters():
            q.grad = None
        xi = x.clone().requires_grad_()
        torch.cuda.synchronize()
        start = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out = m(xi)
        out.backward(dy)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - start
        return out.detach(), xi.grad, [q.grad for q in m.parameters()], peak

    ob, gxb, gwb, peak_b = step(base)
    orr, gxr, gwr, peak_r = step(rec)
    tol = 1e-6 if dtype == torch.float32 else 1e-2
    assert _rel_gpu(orr, ob) < tol
    assert _rel_gpu(gxr, gxb) < tol
    for a, b in zip(gwr, gwb):
        assert _rel_gpu(a, b) < tol
    h_bytes = tokens * inter * torch.finfo(dtype).bits // 8
    assert peak_b - peak_r >= h_bytes // 2, (peak_b, peak_r, h_bytes)


def test_recompute_activation_refusals(fn):
    with pytest.raises(ValueError, match="recompute_activation"):
        fn.GatedMLP(8, 12, fused_gate_up=False, recompute_activation=True)
    with pytest.raises(ValueError, match="recompute_activation"):
        fn.GatedMLP(8, 12, fused_epilogue=True, recompute_activation=True)
