"""CPU tests of the C-ABI boundary: the library loads, exports every function
that include/twell.h declares, and maps bad arguments to status codes before
any HIP call (so none of these touches a GPU)."""
import ctypes
import os

import pytest

from activation_sparse_feedforward_amd import twell as T
from _helpers import header_symbols

pytestmark = pytest.mark.skipif(not os.path.exists(T.LIB_PATH), reason="libtwell.so not built")


def test_exports_every_header_symbol():
    lib = T.library()
    syms = header_symbols()
    assert "twell_pack" in syms and "twell_ffn_fwd" in syms
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(T.EXPORTED)


def _st(**kw):
    base = dict(T=256, d_model=512, d_ff=1024, tile_n=128, slots=16, dtype=T.TWELL_BF16)
    base.update(kw)
    d = T.CDesc(base["T"], base["d_model"], base["d_ff"], base["tile_n"], base["slots"], base["dtype"])
    return T.library().twell_sizes(ctypes.byref(d), ctypes.c_int64(0), ctypes.byref(T.CSizes()))


@pytest.mark.parametrize("kw,code", [
    ({}, T.TWELL_OK),
    ({"T": 0}, T.TWELL_OK),
    ({"T": -1}, T.TWELL_EINVAL),
    ({"d_model": 0}, T.TWELL_EINVAL),
    ({"d_ff": 1000}, T.TWELL_EINVAL),          # not a multiple of tile_n
    ({"slots": 0}, T.TWELL_EINVAL),
    ({"slots": 129}, T.TWELL_EINVAL),           # more slots than tile columns
    ({"dtype": 7}, T.TWELL_EINVAL),
    ({"tile_n": 32, "d_ff": 1024}, T.TWELL_EUNSUPPORTED),
    ({"d_model": 768}, T.TWELL_EUNSUPPORTED),   # bf16 needs d_model % 512 == 0
    ({"d_model": 8192}, T.TWELL_EUNSUPPORTED),
    ({"dtype": T.TWELL_FP32, "d_model": 256}, T.TWELL_OK),
    ({"dtype": T.TWELL_FP32, "d_model": 4096}, T.TWELL_EUNSUPPORTED),
    ({"T": 1 << 40}, T.TWELL_EUNSUPPORTED),      # index space
])
def test_descriptor_validation(kw, code):
    assert _st(**kw) == code


def test_sizes_values():
    s = T.sizes(T.Desc(16384, 2048, 8192, 128, 16, "bf16"))
    assert s["count"] == 16384 * 64 * 4
    assert s["idx"] == 16384 * 64 * 16
    assert s["val"] == 16384 * 64 * 16 * 2
    assert s["ws_dense_fwd"] == 16384 * 8192 * 2 + 2048 * 8192 * 2  # h, then W_down^T
    assert s["ws_pack_classic"] == 16384 * 8192 * 2                    # dense ReLU(g)
    h = T.sizes(T.Desc(16384, 2048, 8192, 128, 16, "bf16"), max_dense_rows=1000)
    assert h["ws_hybrid"] >= 1000 * 8192 * 2 + 64 * 4
    d = T.Desc(16, 512, 1024, 128, 16, "bf16").c()
    assert T.library().twell_sizes(ctypes.byref(d), ctypes.c_int64(-1), ctypes.byref(T.CSizes())) == T.TWELL_EINVAL


def test_null_and_misaligned_pointers_rejected_before_launch():
    lib = T.library()
    d = T.Desc(64, 512, 1024, 128, 16, "bf16").c()
    act = T.CAct(0x1000, 0x2000, 0x3000)
    P = 0x10000
    assert lib.twell_pack(ctypes.byref(d), None, P, act, None, None, None) == T.TWELL_EINVAL
    assert lib.twell_pack(ctypes.byref(d), P + 8, P, act, None, None, None) == T.TWELL_EINVAL
    assert lib.twell_pack(ctypes.byref(d), P, P, T.CAct(0, 0x2000, 0x3000), None, None, None) == T.TWELL_EINVAL
    assert lib.twell_pack(ctypes.byref(d), P, P, act, P + 4, None, None) == T.TWELL_EINVAL  # stats not 8-aligned
    assert lib.twell_ffn_fwd(ctypes.byref(d), P, act, P, P, None, None) == T.TWELL_EINVAL
    assert lib.twell_dense_ffn_fwd(ctypes.byref(d), P, P, P, P, P, P, 100, None) == T.TWELL_EINVAL  # ws too small
    assert lib.twell_dense_ffn_fwd(ctypes.byref(d), P, P, P, P, P, None, 1 << 30, None) == T.TWELL_EINVAL
    assert lib.twell_pack(None, P, P, act, None, None, None) == T.TWELL_EINVAL
    assert lib.twell_pack_classic(ctypes.byref(d), P, P, act, P, 100, None) == T.TWELL_EINVAL  # ws too small
    assert lib.twell_pack_classic(ctypes.byref(d), P, P, act, None, 1 << 30, None) == T.TWELL_EINVAL
    assert lib.twell_pack_classic(ctypes.byref(d), P, P + 2, act, P, 1 << 30, None) == T.TWELL_EINVAL
    r = T.CRoute(P, P, P, P, 10)
    assert lib.twell_ffn_fwd_hybrid(ctypes.byref(d), P, P, act, P, P, P, None, P, 1 << 30, None) == T.TWELL_EINVAL
    assert lib.twell_ffn_fwd_hybrid(ctypes.byref(d), P, P, act, P, P, P, ctypes.byref(r), P, 16, None) == T.TWELL_EINVAL
    r0 = T.CRoute(P, 0, P, P, 10)  # capacity without a dense_rows array
    assert lib.twell_ffn_fwd_hybrid(ctypes.byref(d), P, P, act, P, P, P, ctypes.byref(r0), P, 1 << 30, None) == T.TWELL_EINVAL


def test_noalloc_host_checks_before_any_hip_call():
    """The allocation-free hybrid forward validates like the workspace entry
    point, and refuses a problem whose workspace exceeds its static scratch
    (TWELL_ESCRATCH) before any HIP call."""
    lib = T.library()
    act = T.CAct(0x1000, 0x2000, 0x3000)
    P = 0x10000
    big = T.Desc(16384, 2048, 8192, 128, 16, "bf16")
    assert T.sizes(big, 1024)["ws_hybrid"] > T.NOALLOC_SCRATCH_BYTES
    r = T.CRoute(P, P, P, P, 1024)
    f = lib.twell_ffn_fwd_hybrid_noalloc
    assert f(ctypes.byref(big.c()), P, P, act, P, P, P, ctypes.byref(r), None) == T.TWELL_ESCRATCH
    assert f(ctypes.byref(big.c()), P, P, act, P, P, P, None, None) == T.TWELL_EINVAL
    assert f(ctypes.byref(big.c()), P, P + 2, act, P, P, P, ctypes.byref(r), None) == T.TWELL_EINVAL
    assert f(None, P, P, act, P, P, P, ctypes.byref(r), None) == T.TWELL_EINVAL
    r0 = T.CRoute(P, 0, P, P, 10)  # capacity without a dense_rows array
    assert f(ctypes.byref(big.c()), P, P, act, P, P, P, ctypes.byref(r0), None) == T.TWELL_EINVAL
    e = T.Desc(0, 2048, 8192, 128, 16, "bf16")
    assert f(ctypes.byref(e.c()), None, None, T.CAct(0, 0, 0), None, None, None, ctypes.byref(r), None) == T.TWELL_OK
    assert "scratch" in T.status_str(T.TWELL_ESCRATCH)


def test_empty_batch_is_a_noop():
    lib = T.library()
    d = T.Desc(0, 512, 1024, 128, 16, "bf16").c()
    # T == 0: returns OK without reading any pointer (NULLs are fine)
    assert lib.twell_pack(ctypes.byref(d), None, None, T.CAct(0, 0, 0), None, None, None) == T.TWELL_OK
    assert lib.twell_ffn_fwd(ctypes.byref(d), None, T.CAct(0, 0, 0), None, None, None, None) == T.TWELL_OK
    assert lib.twell_dense_ffn_fwd(ctypes.byref(d), None, None, None, None, None, None, 0, None) == T.TWELL_OK
    assert lib.twell_pack_classic(ctypes.byref(d), None, None, T.CAct(0, 0, 0), None, 0, None) == T.TWELL_OK


def test_status_strings():
    for c in range(5):
        assert T.status_str(c)
    assert "unknown" in T.status_str(99)


def test_binding_refuses_host_tensors():
    import torch
    d = T.Desc(4, 512, 1024, 128, 16, "bf16")
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    act = T.alloc_act(d, device="cpu")
    with pytest.raises(ValueError):
        T.twell_pack(d, x, torch.zeros(1024, 512, dtype=torch.bfloat16), act, stream=0)
