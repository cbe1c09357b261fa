"""MI355X-native forward pass of a top-k Mixture-of-Experts SwiGLU FFN layer.

The computation lives in libmoe.so (hand-written HIP for gfx950 behind the C
ABI in include/moe.h); `binding` marshals torch tensors into it.  Import
`mixture_experts_layer_13_amd.binding` to use it: the import fails loudly
when the library has not been built."""
__all__ = ["binding"]
