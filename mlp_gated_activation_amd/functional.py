"""Autograd functions and a gated-MLP module over the C ABI.

"Kernel Profile: SwiGLU (Tier 1 -- Element-wise)":
  * Identity: an autograd function (forward c = silu(a) * b), a functional
    entry point and an MLP module;
  * Backward Pass / Key Patterns: only a and b are saved, the sigmoid is
    recomputed, and the gradients are written over the saved a and b;
  * Module Parameters: gate, up and down projections without bias.
"Write a Triton SiLU-Mul (SwiGLU) Kernel", Purpose: the MLP is
down_proj(act(gate_proj(x)) * up_proj(x)), optionally with gate and up fused
into one projection whose output is [gate | up] (Inputs, item 4).

Every element of the activation and its gradient is computed by libglu.so;
this module only wires it into autograd.  The projections are ordinary
torch.nn.Linear layers (hipBLASLt GEMMs on ROCm).

In-place backward (the default, as in the profile above): the gradient
overwrites the saved activation inputs, which therefore must not be used by
anything else after the backward.  Pass inplace_backward=False to keep them.

Operands in other layouts (transposed or sliced activations, broadcast
incoming gradients such as the one of ``y.sum()``) go to the strided entry
points without a copy ("Write a Triton SiLU-Mul (SwiGLU) Kernel", Common
failure modes: thread the strides through instead of silently reading a
transposed view); only views whose leading dimensions cannot be merged into
one are copied to a contiguous tensor first.
"""
from __future__ import annotations

import torch
import torch.nn as nn

from . import glu as _glu

_KINDS = ("silu", "gelu_erf", "gelu_tanh", "relu")

# The fused gate/up kernel's few-token tile configuration (csrc/gemm_internal.h:
# kGemmTiles[kGemmSmall] and kGemmSmallMaxM): 128 tokens x 64 features per
# workgroup, taken for at most 256 tokens.
_SMALL_TILE_TOKENS, _SMALL_TILE_FEATURES, _SMALL_MAX_TOKENS = 128, 64, 256
_cu_count = {}


def fused_epilogue_wins(tokens: int, intermediate: int, device) -> bool:
    """Whether the fused gate/up kernel measured faster than the library GEMM
    followed by the activation kernel, for this many tokens and this
    intermediate width.  At few tokens both stream the weights once; the
    fused kernel wins when its few-token tiles fill at most one round of
    workgroups, one per compute unit, and loses when a second, partial
    round follows (bf16, fused / unfused us at 1 .. 256 tokens, hidden x I:
    4096 x 14336 1.02-1.23x up to 128 tokens, 224 workgroups, 0.80x at 256
    with 448; 2048 x 8192 1.04-1.29x up to 256, at most 256 workgroups;
    3584 x 18944 0.72-0.85x, 296 workgroups; 8192 x 28672 0.62-0.99x, 448)."""
    if tokens <= 0 or tokens > _SMALL_MAX_TOKENS:
        return False
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _cu_count:
        _cu_count[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
    tiles = -(-tokens // _SMALL_TILE_TOKENS) * -(-intermediate // _SMALL_TILE_FEATURES)
    return tiles <= _cu_count[idx]
# Hugging Face activation names (a config's hidden_act) -> kinds: "gelu" is
# the exact erf form; "gelu_new" and "gelu_pytorch_tanh" are the tanh form.
HF_ACTIVATIONS = {"silu": "silu", "swish": "silu", "gelu": "gelu_erf", "gelu_new": "gelu_tanh",
                  "gelu_pytorch_tanh": "gelu_tanh", "relu": "relu"}


def _row_major(t: torch.Tensor) -> bool:
    """True when glu_fwd / glu_bwd take t as it is: last dimension contiguous
    and leading dimensions merging into rows at least a row apart."""
    if t.dim() == 0 or (t.shape[-1] > 1 and t.stride(-1) != 1):
        return False
    try:
        v = t.view(-1, t.shape[-1])
    except RuntimeError:
        return False
    return v.shape[0] <= 1 or v.stride(0) >= v.shape[1]


def _writable(t: torch.Tensor) -> bool:
    """t can take a result in place: it merges into 2-D and no two of its
    elements share memory (no stride 0 along a dimension of size > 1)."""
    return _viewable(t) is t and all(st != 0 for n, st in zip(t.shape, t.stride()) if n > 1)


def _viewable(t: torch.Tensor) -> torch.Tensor:
    """t itself when its leading dimensions merge into one (any strides: the
    strided entry points take transposed, sliced and broadcast views), else a
    contiguous copy (this allocates)."""
    if t.dim() == 0:
        return t   # rejected by the binding: the activation needs a dimension
    try:
        t.view(-1, t.shape[-1])
        return t
    except RuntimeError:
        return t.contiguous()


class GatedActivation(torch.autograd.Function):
    """y = act(a) * b for separate a, b."""

    @staticmethod
    def forward(ctx, a, b, kind: str, inplace_backward: bool):
        if _row_major(a) and _row_major(b):
            y = _glu.glu_fwd(kind, "separate", a, b)
        else:
            y = _glu.glu_fwd_strided(kind, _viewable(a), _viewable(b))
        ctx.save_for_backward(a, b)
        ctx.kind = kind
        ctx.inplace_backward = inplace_backward
        return y

    @staticmethod
    def backward(ctx, dy):
        a, b = ctx.saved_tensors
        inplace = ctx.inplace_backward
        if _row_major(a) and _row_major(b) and _row_major(dy):
            if inplace:
                _glu.glu_bwd(ctx.kind, "separate", a, b, dy, inplace=True)
                return a, b, None, None
            da, db = _glu.glu_bwd(ctx.kind, "separate", a, b, dy, inplace=False)
            return da, db, None, None
        dy = _viewable(dy)
        if inplace and _writable(a) and _writable(b):
            _glu.glu_bwd_strided(ctx.kind, a, b, dy, da=a, db=b)
            return a, b, None, None
        da, db = _glu.glu_bwd_strided(ctx.kind, _viewable(a), _viewable(b), dy)
        return da, db, None, None


class FusedGatedActivation(torch.autograd.Function):
    """y = act(x[..., :I]) * x[..., I:] for the fused [gate | up] layout."""

    @staticmethod
    def forward(ctx, x, kind: str, inplace_backward: bool):
        if _row_major(x):
            y = _glu.glu_fwd(kind, "gate_up", x)
        else:
            if x.shape[-1] % 2:
                raise ValueError(f"gate_up input width {x.shape[-1]} is odd")
            xv = _viewable(x)
            i = x.shape[-1] // 2
            y = _glu.glu_fwd_strided(kind, xv[..., :i], xv[..., i:])
        ctx.save_for_backward(x)
        ctx.kind = kind
        ctx.inplace_backward = inplace_backward
        return y

    @staticmethod
    def backward(ctx, dy):
        (x,) = ctx.saved_tensors
        inplace = ctx.inplace_backward
        if _row_major(x) and _row_major(dy):
            if inplace:
                _glu.glu_bwd(ctx.kind, "gate_up", x, None, dy, inplace=True)
                return x, None, None
            dx = _glu.glu_bwd(ctx.kind, "gate_up", x, None, dy, inplace=False)
            return dx, None, None
        dy = _viewable(dy)
        i = x.shape[-1] // 2
        if inplace and _writable(x):
            _glu.glu_bwd_strided(ctx.kind, x[..., :i], x[..., i:], dy, da=x[..., :i], db=x[..., i:])
            return x, None, None
        xv = _viewable(x)
        dx = torch.empty_like(xv)
        _glu.glu_bwd_strided(ctx.kind, xv[..., :i], xv[..., i:], dy, da=dx[..., :i], db=dx[..., i:])
        return dx, None, None


class FusedGateUpActivation(torch.autograd.Function):
    """h = act(x @ Wg^T) * (x @ Wu^T) for a fused [gate | up] weight w of
    shape (2I, H), with the activation in the GEMM epilogue ("Fused Kernels",
    section 4).  The forward keeps the pre-activations [g | u] (written by
    the same kernel) for the backward, which runs the elementwise backward
    on them in place ("Kernel Profile: SwiGLU", Backward Pass) and then the
    two GEMMs of the projection's gradient: dx = d[g|u] @ w and
    dw = d[g|u]^T @ x (torch matmuls)."""

    @staticmethod
    def forward(ctx, x, w, kind: str):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        need = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        if need:
            h, gu = _glu.glu_gemm_fwd(kind, x2, w, gu=True)
            ctx.save_for_backward(x2, w, gu)
        else:
            h = _glu.glu_gemm_fwd(kind, x2, w)
        ctx.kind = kind
        ctx.lead = lead
        return h.reshape(*lead, h.shape[-1])

    @staticmethod
    def backward(ctx, dh):
        x2, w, gu = ctx.saved_tensors
        dh2 = dh.reshape(-1, dh.shape[-1])
        if not _row_major(dh2):
            dh2 = dh2.contiguous()
        dgu = _glu.glu_bwd(ctx.kind, "gate_up", gu, None, dh2, inplace=True)
        dx = torch.mm(dgu, w) if ctx.needs_input_grad[0] else None
        dw = torch.mm(dgu.t(), x2) if ctx.needs_input_grad[1] else None
        if dx is not None:
            dx = dx.reshape(*ctx.lead, dx.shape[-1])
        return dx, dw, None


class ActDownRecompute(torch.autograd.Function):
    """out = (act(gu[..., :I]) * gu[..., I:]) @ w_down^T, keeping only gu for
    the backward: h is recomputed there from gu (one more activation pass)
    instead of being kept for the down projection's weight gradient, the
    same trade the kernels make for the sigmoid ("Kernel Profile: SwiGLU",
    Key Patterns: recomputation over saving).  The backward then runs the
    elementwise backward in place over gu, as FusedGatedActivation does."""

    @staticmethod
    def forward(ctx, gu, w_down, kind: str):
        lead = gu.shape[:-1]
        gu2 = gu.reshape(-1, gu.shape[-1])
        if not _row_major(gu2):
            gu2 = gu2.contiguous()
        h = _glu.glu_fwd(kind, "gate_up", gu2)
        out = torch.mm(h, w_down.t())
        ctx.save_for_backward(gu2, w_down)
        ctx.kind = kind
        ctx.lead = lead
        return out.reshape(*lead, out.shape[-1])

    @staticmethod
    def backward(ctx, dout):
        gu2, w_down = ctx.saved_tensors
        dout2 = dout.reshape(-1, dout.shape[-1])
        dw = None
        if ctx.needs_input_grad[1]:
            h = _glu.glu_fwd(ctx.kind, "gate_up", gu2)
            dw = torch.mm(dout2.t(), h)
            del h
        dgu = None
        if ctx.needs_input_grad[0]:
            dh = torch.mm(dout2, w_down)
            dgu = _glu.glu_bwd(ctx.kind, "gate_up", gu2, None, dh, inplace=True)
            dgu = dgu.reshape(*ctx.lead, dgu.shape[-1])
        return dgu, dw, None


def gate_up_activation(x: torch.Tensor, w: torch.Tensor, kind: str = "silu") -> torch.Tensor:
    """act(x @ w[:I]^T) * (x @ w[I:]^T) for a fused [gate | up] weight w of
    shape (2I, H), on the matrix cores with the activation in the epilogue."""
    if kind not in _KINDS:
        raise ValueError(f"unknown kind {kind!r}; expected one of {_KINDS}")
    return FusedGateUpActivation.apply(x, w, kind)


def gated_activation(a: torch.Tensor, b: torch.Tensor | None = None, kind: str = "silu",
                     inplace_backward: bool = True) -> torch.Tensor:
    """act(a) * b; with b None, a is the fused [gate | up] tensor."""
    if kind not in _KINDS:
        raise ValueError(f"unknown kind {kind!r}; expected one of {_KINDS}")
    if b is None:
        return FusedGatedActivation.apply(a, kind, inplace_backward)
    return GatedActivation.apply(a, b, kind, inplace_backward)


def swiglu(a, b=None, inplace_backward: bool = True):
    """silu(a) * b (SwiGLU)."""
    return gated_activation(a, b, "silu", inplace_backward)


def geglu(a, b=None, approximate: str = "none", inplace_backward: bool = True):
    """gelu(a) * b (GeGLU); approximate 'none' (erf form) or 'tanh'."""
    if approximate not in ("none", "tanh"):
        raise ValueError("approximate must be 'none' or 'tanh'")
    return gated_activation(a, b, "gelu_erf" if approximate == "none" else "gelu_tanh", inplace_backward)


def reglu(a, b=None, inplace_backward: bool = True):
    """relu(a) * b (ReGLU)."""
    return gated_activation(a, b, "relu", inplace_backward)


class GatedMLP(nn.Module):
    """down_proj(act(gate_proj(x)) * up_proj(x)) with the activation step on
    the gfx950 kernels.  fused_gate_up=True keeps gate and up as one
    projection of width 2*intermediate_size whose output is [gate | up].
    recompute_activation=True (with fused_gate_up) keeps only [gate | up]
    for the backward and recomputes act(gate) * up there (ActDownRecompute),
    saving one tokens x intermediate_size activation per layer for one more
    activation pass.
    fused_epilogue=True (needs fused_gate_up, bf16/fp16) computes that
    projection and the activation in one kernel (gate_up_activation).
    fused_epilogue="auto" (the default) does so only where that kernel
    measured faster than the library GEMM followed by the separate activation
    kernel (fused_epilogue_wins: few tokens, and few enough workgroups for
    one round; at 4096 tokens the unfused path is 1.1x faster), with bf16 or
    fp16 operands that meet its alignment (see uses_fused_epilogue)."""

    def __init__(self, hidden_size: int, intermediate_size: int, kind: str = "silu",
                 fused_gate_up: bool = True, inplace_backward: bool = True, fused_epilogue="auto",
                 recompute_activation: bool = False, device=None, dtype=None):
        super().__init__()
        if kind not in _KINDS:
            raise ValueError(f"unknown kind {kind!r}")
        if fused_epilogue not in (True, False, "auto"):
            raise ValueError("fused_epilogue must be True, False or 'auto'")
        if fused_epilogue is True and not fused_gate_up:
            raise ValueError("fused_epilogue needs fused_gate_up=True")
        if recompute_activation and (not fused_gate_up or fused_epilogue is True):
            raise ValueError("recompute_activation needs fused_gate_up=True and fused_epilogue=False")
        self.recompute_activation = recompute_activation
        self.kind = kind
        self.fused_gate_up = fused_gate_up
        self.fused_epilogue = fused_epilogue
        self.inplace_backward = inplace_backward
        kw = dict(bias=False, device=device, dtype=dtype)
        if fused_gate_up:
            self.gate_up_proj = nn.Linear(hidden_size, 2 * intermediate_size, **kw)
        else:
            self.gate_proj = nn.Linear(hidden_size, intermediate_size, **kw)
            self.up_proj = nn.Linear(hidden_size, intermediate_size, **kw)
        self.down_proj = nn.Linear(intermediate_size, hidden_size, **kw)

    @classmethod
    def from_config(cls, config, **kwargs) -> "GatedMLP":
        """Build from a Hugging Face model config ("Kernel Profile: SwiGLU",
        Module Parameters: the module takes the model config): its
        hidden_size, intermediate_size and hidden_act, which must be one of
        HF_ACTIVATIONS.  A config with mlp_bias set is refused (the
        projections here have no bias).  kwargs go to the constructor."""
        act = getattr(config, "hidden_act", "silu")
        if act not in HF_ACTIVATIONS:
            raise ValueError(f"hidden_act {act!r} is not a gated activation this module computes; "
                             f"expected one of {sorted(HF_ACTIVATIONS)}")
        if getattr(config, "mlp_bias", False):
            raise ValueError("mlp_bias=True: the gate, up and down projections here have no bias")
        return cls(config.hidden_size, config.intermediate_size, HF_ACTIVATIONS[act], **kwargs)

    def _load_from_state_dict(self, state_dict, prefix, *args, **kwargs):
        # A state dict with separate gate and up weights (the Hugging Face
        # layout, gate_proj / up_proj / down_proj) loads into the fused
        # [gate | up] projection: gate rows first, then up rows.
        g, u = prefix + "gate_proj.weight", prefix + "up_proj.weight"
        if self.fused_gate_up and g in state_dict and u in state_dict:
            state_dict[prefix + "gate_up_proj.weight"] = torch.cat([state_dict.pop(g), state_dict.pop(u)], 0)
        super()._load_from_state_dict(state_dict, prefix, *args, **kwargs)

    def uses_fused_epilogue(self, x: torch.Tensor) -> bool:
        """Whether forward(x) runs the gate/up projection with the activation
        fused into its epilogue."""
        if self.fused_epilogue is not True and self.fused_epilogue != "auto":
            return False
        if self.fused_epilogue is True:
            return True
        # "auto"
        if not self.fused_gate_up or self.recompute_activation:
            return False
        w = self.gate_up_proj.weight
        H = x.shape[-1]
        if not (x.is_cuda and x.dtype in (torch.bfloat16, torch.float16) and w.dtype == x.dtype
                and w.device == x.device and H % 8 == 0 and H > 0):
            return False
        if not fused_epilogue_wins(x.numel() // H, w.shape[0] // 2, x.device):
            return False
        # the kernel's operand rules: 16-byte aligned rows, row strides a multiple of 8
        x2 = x.reshape(-1, H)
        return (x2.stride(-1) == 1 and x2.stride(0) % 8 == 0 and x2.data_ptr() % 16 == 0
                and w.stride(-1) == 1 and w.stride(0) % 8 == 0 and w.data_ptr() % 16 == 0)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.uses_fused_epilogue(x):
            return self.down_proj(gate_up_activation(x, self.gate_up_proj.weight, self.kind))
        if self.recompute_activation:
            return ActDownRecompute.apply(self.gate_up_proj(x), self.down_proj.weight, self.kind)
        if self.fused_gate_up:
            h = gated_activation(self.gate_up_proj(x), None, self.kind, self.inplace_backward)
        else:
            h = gated_activation(self.gate_proj(x), self.up_proj(x), self.kind, self.inplace_backward)
        return self.down_proj(h)
