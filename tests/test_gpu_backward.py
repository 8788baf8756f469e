"""GPU parity of the backward (twell_ffn_bwd) against the oracle's manual
backward, through the C ABI.

The activation mask is taken from the kernels under test, so that both sides
decide g > 0 the same way: for rows served from TwELL, the stored slots (the
forward's own TwELL, itself checked bit-exact elsewhere); for dense-fallback
rows, the gate kernel's dense debug output.  Values (g, u, h, ...) are the
oracle's own float64 ones.  Each of dx, dW_gate^T, dW_up^T, dW_down must lie
within 1e-2 * max|ref| (fp32: 1e-5) of the oracle.
"""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from oracle import twell_oracle as O
from _helpers import assert_rows_written, check_guards, desc_for, dev, guarded, host64, poison_, say, within

pytestmark = pytest.mark.gpu
TOL = {"fp32": 1e-5, "bf16": 1e-2}


def run_bwd(w, cap, l1=2e-5, label="", check=True):
    say(f"[gpu case] backward {label} {w.name} T={w.T} cap={cap} l1={l1}")
    inp = W.make_inputs(w, with_dy=True)
    desc = desc_for(w)
    x, wg, wu, wd, dy = (dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down", "dy"))
    act = T.alloc_act(desc)
    gate = torch.empty((w.T, w.d_ff), dtype=desc.torch_dtype, device="cuda")
    T.twell_pack(desc, x, wg, act, gate_dbg=gate)
    route = T.alloc_route(desc, cap)
    y = torch.empty((w.T, w.d_model), dtype=desc.torch_dtype, device="cuda")
    ws = torch.empty(T.sizes(desc, cap)["ws_hybrid"], dtype=torch.uint8, device="cuda")
    T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y, route, ws)
    wsb = guarded((T.sizes(desc, cap)["ws_bwd"],), torch.uint8)
    dx = guarded((w.T, w.d_model), desc.torch_dtype)
    dws = [guarded((w.d_ff, w.d_model), torch.float32) for _ in range(3)]
    T.twell_ffn_bwd(desc, x, act, route, wg, wu, wd, dy, l1, dx, *dws, wsb)
    torch.cuda.synchronize()
    check_guards(wsb, dx, *dws)
    assert_rows_written(dx, "dx")
    for name, t in zip(("dw_gate_t", "dw_up_t", "dw_down"), dws):
        assert_rows_written(t, name)
    out = dict(dx=dx, dws=dws, act=act, route=route, desc=desc, tensors=(x, wg, wu, wd, dy), wsb=wsb, gate=gate)
    if not check:
        return out
    count = act.count.cpu().numpy()
    idx = act.idx.cpu().numpy()
    val = host64(act.val)
    n_ell, n_dense, _ = route.n_rows.cpu().numpy().tolist()
    ell = route.ell_rows.cpu().numpy()[:n_ell]
    dns = route.dense_rows.cpu().numpy()[:n_dense] if cap else np.zeros(0, np.int64)
    mask = np.zeros((w.T, w.d_ff), bool)
    mask[ell] = O.twell_unpack(count[ell], idx[ell], val[ell], w.tile_n) != 0
    mask[dns] = host64(gate)[dns] > 0
    ref = O.ffn_backward(inp["x"], inp["w_gate_t"], inp["w_up_t"], inp["w_down"], inp["dy"], l1, active=mask)
    tol = TOL[w.dtype]
    got = {"dx": host64(dx), "dw_gate_t": host64(dws[0]), "dw_up_t": host64(dws[1]), "dw_down": host64(dws[2])}
    for k, v in got.items():
        within(v, ref[k], tol, f"{w.name} T={w.T} {w.dtype}: {k} vs oracle backward")
    say(f"   ok: n_ell={n_ell} n_dense={n_dense} pairs={int(mask[ell].sum())}")
    return out


@pytest.mark.parametrize("T_,cap", [(600, 256), (257, 300), (64, 64)])
def test_backward_lognormal(T_, cap):
    run_bwd(W.workload(4, T=T_), cap, label="lognormal")


def test_backward_all_ell():
    run_bwd(W.workload(3, T=530), 0, label="uniform cap=0")


def test_backward_cap_exceeded():
    r = run_bwd(W.workload(5, T=400, rho=0.05), 2, label="cap=2")
    assert int(r["route"].n_rows[2]) > 0


def test_backward_all_dense():
    r = run_bwd(W.workload(5, T=300, rho=0.3), 300, label="all dense")
    assert int(r["route"].n_rows[0]) == 0


def test_backward_large_l1():
    run_bwd(W.workload(4, T=300), 300, l1=0.05, label="l1=0.05")


def test_backward_fp32():
    import dataclasses
    w = dataclasses.replace(W.workload(1), slots=2)
    run_bwd(w, 256, label="fp32 C=2")


def test_backward_wide_rows():
    """d_model = 4096 (bf16), the widest rows the library takes, at 160 rows:
    the dx pass runs one wave per ELL row (the lockstep workgroups take wide
    rows from 4096 rows on)."""
    import dataclasses
    w = dataclasses.replace(W.workload(4, T=160), d_model=4096)
    run_bwd(w, 64, label="d_model=4096")


def test_backward_wide_rows_lockstep():
    """d_model = 4096 at 4096 lognormal rows: the light rows' dx in the 8-wave
    lockstep workgroups (two rows per wave), the heavy rows cut into tile
    ranges, all outputs against the oracle."""
    run_bwd(W.workload(4, T=4096, d_model=4096, d_ff=8192), 256, label="d_model=4096 lockstep")


def test_backward_wide_ff():
    """d_ff = 16384: the pair transpose's per-block row masks span two
    8192-neuron chunks."""
    run_bwd(W.workload(4, T=200, d_model=512, d_ff=16384), 64, label="d_ff=16384")


def test_backward_deterministic():
    w = W.workload(4, T=900)
    a = run_bwd(w, 512, label="det a", check=False)
    desc, (x, wg, wu, wd, dy) = a["desc"], a["tensors"]
    dx2 = torch.empty_like(a["dx"])
    dws2 = [torch.empty_like(t) for t in a["dws"]]
    T.twell_ffn_bwd(desc, x, a["act"], a["route"], wg, wu, wd, dy, 2e-5, dx2, *dws2, a["wsb"])
    torch.cuda.synchronize()
    assert torch.equal(a["dx"].view(torch.int16), dx2.view(torch.int16))
    for u, v in zip(a["dws"], dws2):
        assert torch.equal(u, v)


def test_backward_empty_batch():
    w = W.workload(4, T=16)
    desc = desc_for(w, T=0)
    route = T.alloc_route(desc, 4)
    act = T.alloc_act(desc)
    ws = torch.empty(T.sizes(desc, 4)["ws_bwd"], dtype=torch.uint8, device="cuda")
    wmat = torch.zeros((w.d_ff, w.d_model), dtype=torch.bfloat16, device="cuda")
    dws = [poison_(torch.empty((w.d_ff, w.d_model), dtype=torch.float32, device="cuda")) for _ in range(3)]
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    T.twell_ffn_bwd(desc, e, act, route, wmat, wmat, wmat, e, 2e-5, e, *dws, ws)
    torch.cuda.synchronize()
    for t in dws:
        assert torch.all(t == 0)


def test_backward_full_size():
    """The training workload at full size (T=16384, d=2048, F=8192), all outputs."""
    run_bwd(W.workload(4), 1024, label="full c4")
