"""TPLA decode attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libtpla.so`` (hand-written HIP
kernels); ``tensor_latent_decode_amd.tpla`` is its thin Python binding.
Importing this package does not load the library; the first call does, and
fails loudly if it is missing.
"""

__version__ = "0.4.0"
