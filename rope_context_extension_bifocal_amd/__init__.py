"""Dynamic Bifocal RoPE attention (Jet-Long) for AMD MI355X.

The compute path is the HIP library libbifocal.so (include/bifocal.h); the
`bifocal` module is its ctypes binding and `workloads` holds the seeded
synthetic inputs. Import `rope_context_extension_bifocal_amd.bifocal` to use
the kernels.
"""
