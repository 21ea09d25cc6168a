"""MI355X-native sparse mixture-of-experts layer (router, permute, grouped
SwiGLU expert FFN, combine) behind a C-ABI HIP library.

The compute path is ``libmoe.so`` (hand-written HIP kernels for gfx950);
``expert_ffn_layer_amd.moe`` is its thin ctypes binding.  Importing the
package does not load the library; the first call into the binding does,
and raises if it is missing.
"""
