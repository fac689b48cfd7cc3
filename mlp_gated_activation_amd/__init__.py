"""MI355X-native fused gated activation y = act(a) * b (SwiGLU, GeGLU, ReGLU).

The compute path is the C-ABI library ``libglu.so`` (hand-written HIP
kernels for gfx950); ``mlp_gated_activation_amd.glu`` is its thin Python
binding.  Importing this package does not load the library; importing
``glu`` does, and fails loudly if it has not been built.
"""
__all__ = ["glu", "inputs"]
