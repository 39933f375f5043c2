"""fa_fwd: a FlashAttention-2 forward pass for AMD MI355X (gfx950), in HIP.

The compute path is the C-ABI library libfa_fwd.so (hand-written HIP kernels);
`exact_attention_17_amd.fa` is the thin ctypes binding over it.  Importing the
package does not load the library; `from exact_attention_17_amd import fa` does.
"""
__all__ = ["fa", "inputs", "metrics"]
