"""GatedMLP built from a Hugging Face model config, and loading of Hugging
Face's gate_proj / up_proj / down_proj weights ("Kernel Profile: SwiGLU",
Module Parameters).  Construction and state-dict loading run no kernel, so
these run on the CPU; tests/test_gpu_functional.py runs the module."""
from __future__ import annotations

from types import SimpleNamespace

import pytest
import torch

from conftest import ensure_built

ensure_built()
from mlp_gated_activation_amd import functional as F  # noqa: E402


@pytest.mark.parametrize("act,kind", [("silu", "silu"), ("swish", "silu"), ("gelu", "gelu_erf"),
                                      ("gelu_new", "gelu_tanh"), ("gelu_pytorch_tanh", "gelu_tanh"),
                                      ("relu", "relu")])
def test_from_config_activation_names(act, kind):
    m = F.GatedMLP.from_config(SimpleNamespace(hidden_size=8, intermediate_size=12, hidden_act=act))
    assert m.kind == kind
    assert tuple(m.gate_up_proj.weight.shape) == (24, 8)
    assert tuple(m.down_proj.weight.shape) == (8, 12)


def test_from_config_refusals():
    with pytest.raises(ValueError, match="hidden_act"):
        F.GatedMLP.from_config(SimpleNamespace(hidden_size=8, intermediate_size=12, hidden_act="tanh"))
    with pytest.raises(ValueError, match="mlp_bias"):
        F.GatedMLP.from_config(SimpleNamespace(hidden_size=8, intermediate_size=12, hidden_act="silu",
                                               mlp_bias=True))


def test_from_llama_config():
    transformers = pytest.importorskip("transformers")
    cfg = transformers.LlamaConfig(hidden_size=32, intermediate_size=88, hidden_act="silu")
    m = F.GatedMLP.from_config(cfg, fused_gate_up=False)
    assert (m.kind, m.gate_proj.in_features, m.gate_proj.out_features) == ("silu", 32, 88)


@pytest.mark.parametrize("fused", [True, False])
def test_loads_separate_gate_up_weights(fused):
    g = torch.Generator().manual_seed(0)
    sd = {"gate_proj.weight": torch.randn(12, 8, generator=g), "up_proj.weight": torch.randn(12, 8, generator=g),
          "down_proj.weight": torch.randn(8, 12, generator=g)}
    m = F.GatedMLP(8, 12, fused_gate_up=fused)
    m.load_state_dict(dict(sd))
    if fused:
        # gate rows first, then up rows: [gate | up] along the output features
        assert torch.equal(m.gate_up_proj.weight[:12], sd["gate_proj.weight"])
        assert torch.equal(m.gate_up_proj.weight[12:], sd["up_proj.weight"])
        # and the module's own state dict round-trips
        m2 = F.GatedMLP(8, 12, fused_gate_up=True)
        m2.load_state_dict(m.state_dict())
        assert torch.equal(m2.gate_up_proj.weight, m.gate_up_proj.weight)
    else:
        assert torch.equal(m.gate_proj.weight, sd["gate_proj.weight"])
        assert torch.equal(m.up_proj.weight, sd["up_proj.weight"])
    assert torch.equal(m.down_proj.weight, sd["down_proj.weight"])


def test_nested_prefix():
    """The conversion works under a parent module's prefix too."""
    parent = torch.nn.Module()
    parent.mlp = F.GatedMLP(8, 12)
    g = torch.Generator().manual_seed(1)
    sd = {"mlp.gate_proj.weight": torch.randn(12, 8, generator=g), "mlp.up_proj.weight": torch.randn(12, 8, generator=g),
          "mlp.down_proj.weight": torch.randn(8, 12, generator=g)}
    parent.load_state_dict(dict(sd))
    assert torch.equal(parent.mlp.gate_up_proj.weight[12:], sd["mlp.up_proj.weight"])


def test_fused_epilogue_modes():
    """fused_epilogue takes True, False or "auto" (the default); "auto" never
    picks the fused GEMM for CPU tensors, and combines with
    recompute_activation (which then wins)."""
    m = F.GatedMLP(64, 96)
    assert m.fused_epilogue == "auto"
    assert not m.uses_fused_epilogue(torch.randn(4, 64, dtype=torch.bfloat16))
    r = F.GatedMLP(64, 96, recompute_activation=True)
    assert not r.uses_fused_epilogue(torch.randn(4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        F.GatedMLP(64, 96, fused_epilogue="yes")
    with pytest.raises(ValueError):
        F.GatedMLP(64, 96, fused_gate_up=False, fused_epilogue=True)
    F.GatedMLP(64, 96, fused_gate_up=False)   # "auto" needs no fused [gate | up]


def test_fused_epilogue_rule():
    """"auto" takes the fused gate/up kernel for at most 256 tokens whose
    few-token tiles (128 tokens x 64 features) number at most one per
    compute unit; the tile constants mirror the kernel's."""
    import os
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "mlp_gated_activation_amd", "csrc", "gemm_internal.h")).read()
    tiles = re.search(r"kGemmTiles\[2\] = \{\{(\d+), (\d+)\}, \{(\d+), (\d+)\}\}", text)
    assert (F._SMALL_TILE_TOKENS, F._SMALL_TILE_FEATURES) == (int(tiles.group(3)), int(tiles.group(4)))
    assert F._SMALL_MAX_TOKENS == int(re.search(r"#define GLU_GEMM_SMALL_MAX_M (\d+)", text).group(1))
    saved = dict(F._cu_count)
    F._cu_count[0] = 256          # MI355X: 256 compute units (no device here)
    try:
        wins = lambda m, n: F.fused_epilogue_wins(m, n, "cuda:0")
        assert wins(1, 14336) and wins(128, 14336) and not wins(129, 14336)    # 224, then 448 tiles
        assert wins(256, 8192) and not wins(257, 8192)
        assert not wins(16, 18944) and not wins(16, 28672)                     # 296, 448 tiles
        assert wins(16, 64 * 256) and not wins(16, 64 * 256 + 1)
        assert not wins(0, 8192)
    finally:
        F._cu_count.clear()
        F._cu_count.update(saved)
