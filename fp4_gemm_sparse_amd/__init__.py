"""SpliceGEMM on MI355X (gfx950): NVFP4 W4A4 linear layers whose highest-variance
input channels are kept in BF16 (FourSight, arXiv 2611.04887v1, Sec. 4.2 and 5.1).

The compute path is the HIP library libsplice.so (C ABI in include/splice.h);
`fp4_gemm_sparse_amd.splice` is its thin Python binding.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""
__all__ = ["splice", "synth"]
