"""MI355X (gfx950) library for strictly causal second-order Higher-order Linear
Attention: hand-written HIP kernels behind the C ABI in ``include/hla2.h``.

``causal_prefix_scan_hla2_amd.hla2`` is the thin ctypes binding (argument
marshalling only); ``causal_prefix_scan_hla2_amd.inputs`` holds the seeded
synthetic input generators; ``causal_prefix_scan_hla2_amd.build`` compiles the
shared library in-tree.  Submodules are imported lazily so that importing the
package never loads the GPU library by itself.
"""
__all__ = ["hla2", "inputs", "build"]
