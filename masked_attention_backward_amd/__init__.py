"""Masked attention backward for AMD MI355X (gfx950): HIP kernels behind a small C ABI.

Two masked forms of the FlashAttention-style backward pass:
  * GQA attention with a learnable per-head sink logit and a sliding causal window (BHSD);
  * block-sparse MHA driven by a uint8 block mask [B, N, ceil(Sq/bx), ceil(Skv/by)] (BNSD).

``masked_attention_backward_amd.api`` holds the thin torch binding (argument marshalling
only); every step of the computation runs in the HIP library ``libmaskattn.so``.  Importing
the binding fails loudly when that library has not been built.
"""

__all__ = ["api", "workloads"]
