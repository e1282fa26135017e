"""MI355X (gfx950) verify pass of lossless speculative decoding.

The work runs in a C-ABI HIP library (``libdspk.so``, entry points declared in
``include/dspk.h``); this package only marshals torch tensors into its calls
(``speculative_decoding_verify_dspk_amd.binding``) and provides the seeded
synthetic inputs (``speculative_decoding_verify_dspk_amd.inputs``).  The library
is loaded on first use, so the input generators import without a GPU.
"""
__all__ = ["inputs", "binding"]
