"""libflce: fused LM-head linear + cross-entropy (log-prob, LSE, entropy) for gfx950.

`log_prob_amd.flce` is the ctypes binding of the C ABI declared in include/flce.h;
`log_prob_amd.autograd` wraps it as a torch.autograd.Function (linear_logprob).
"""
__all__ = ["flce", "autograd"]
