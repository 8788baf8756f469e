"""TwELL activation-sparse gated FFN for MI355X (gfx950).

The compute path is libtwell.so (HIP kernels + C ABI, include/twell.h); the
Python module ``twell`` is its thin ctypes binding.  ``workloads`` draws the
seeded synthetic inputs.
"""
from .twell import (Act, Desc, Route, TwellError, alloc_act, alloc_route, library, sizes,  # noqa: F401
                    status_str, twell_dense_ffn_fwd, twell_ffn_bwd, twell_ffn_fwd, twell_ffn_fwd_hybrid,
                    twell_pack, twell_pack_classic)
