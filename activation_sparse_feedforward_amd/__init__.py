"""TwELL activation-sparse gated FFN for MI355X (gfx950).

The compute path is libtwell.so (HIP kernels + C ABI, include/twell.h); the
Python module ``twell`` is its thin ctypes binding.  ``workloads`` draws the
seeded synthetic inputs.
"""
from .twell import (Act, Desc, TwellError, alloc_act, library, sizes, status_str,  # noqa: F401
                    twell_dense_ffn_fwd, twell_ffn_fwd, twell_pack)
