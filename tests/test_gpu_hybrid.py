"""GPU parity of the hybrid forward (router + fused TwELL rows + dense MFMA
fallback rows) against the CPU oracle, through the C ABI.

  * route lists, counters and row kinds are exact against the oracle router
    applied to the kernel's own counts (with the dense-row cap applied);
  * y: ELL rows within tol of the oracle's TwELL forward on the kernel's
    TwELL; dense rows within tol of the oracle's dense FFN; and every row
    within tol of the dense FFN when no row exceeds the cap;
  * the canaries around every output buffer and the workspace stay untouched.
"""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from oracle import twell_oracle as O
from _helpers import (assert_rows_written, check_guards, desc_for, dev, guarded, guarded_act, guarded_route, host64,
                      poison_, say, within)

pytestmark = pytest.mark.gpu
TOL = {"fp32": 1e-5, "bf16": 1e-2}


def run_hybrid(w, cap, rows=None, label=""):
    say(f"[gpu case] hybrid {label} {w.name} T={w.T} cap={cap}")
    inp = W.make_inputs(w)
    desc = desc_for(w)
    x, wg, wu, wd = (dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
    act = guarded_act(desc)
    T.twell_pack(desc, x, wg, act)
    route = guarded_route(desc, cap)
    ws = guarded((T.sizes(desc, cap)["ws_hybrid"],), torch.uint8)
    y = guarded((w.T, w.d_model), desc.torch_dtype)
    T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y, route, ws)
    torch.cuda.synchronize()
    check_guards(*act, *route, ws, y)
    assert_rows_written(y, "hybrid y")

    count = act.count.cpu().numpy()
    idx = act.idx.cpu().numpy()
    val = host64(act.val)
    n_rows = route.n_rows.cpu().numpy()
    dense, ell_all, dense_all = O.route(count, w.slots)
    kept = dense_all[:cap]
    over = dense_all[cap:]
    ell_exp = np.sort(np.concatenate([ell_all, over])).astype(np.int32)
    assert n_rows.tolist() == [len(ell_exp), len(kept), len(over)]
    np.testing.assert_array_equal(route.ell_rows.cpu().numpy()[:len(ell_exp)], ell_exp)
    if cap:
        np.testing.assert_array_equal(route.dense_rows.cpu().numpy()[:len(kept)], kept)
    kind = np.zeros(w.T, np.uint8)
    kind[kept] = 1
    np.testing.assert_array_equal(route.row_kind.cpu().numpy()[:w.T], kind)

    yh = host64(y)
    sel = np.arange(w.T) if rows is None else np.asarray(rows)
    sel_ell = np.intersect1d(sel, ell_exp)
    sel_dense = np.intersect1d(sel, kept)
    tol = TOL[w.dtype]
    f = O.ffn_forward(inp["x"][sel], inp["w_gate_t"], inp["w_up_t"], inp["w_down"])
    scale = max(np.abs(f["y"]).max(), 1e-30)
    if sel_ell.size:
        y_ref = O.twell_forward(inp["x"][sel_ell], count[sel_ell], idx[sel_ell], val[sel_ell], w.tile_n,
                                inp["w_up_t"], inp["w_down"])
        within(yh[sel_ell], y_ref, tol, f"hybrid {w.name} T={w.T}: ELL rows vs oracle TwELL forward", scale=scale)
    if sel_dense.size:
        y_ref = O.ffn_forward(inp["x"][sel_dense], inp["w_gate_t"], inp["w_up_t"], inp["w_down"])["y"]
        within(yh[sel_dense], y_ref, tol, f"hybrid {w.name} T={w.T}: dense rows vs oracle dense FFN", scale=scale)
    if len(over) == 0:
        # the hybrid format is exact: every row matches the dense FFN
        within(yh[sel], f["y"], tol, f"hybrid {w.name} T={w.T}: all rows vs oracle dense FFN", scale=scale)
    say(f"   ok: n_ell={n_rows[0]} n_dense={n_rows[1]} over_cap={n_rows[2]}")
    return dict(y=y, route=route, act=act, inp=inp, desc=desc)


@pytest.mark.parametrize("T_,cap", [(1500, 512), (257, 300), (64, 64)])
def test_hybrid_lognormal_tail(T_, cap):
    run_hybrid(W.workload(4, T=T_), cap, label="lognormal")


def test_hybrid_cap_exceeded_routes_rest_to_ell():
    w = W.workload(5, T=600, rho=0.05)   # ~1.5% of rows overflow C=16 at 5% density
    r = run_hybrid(w, 3, label="cap=3")
    assert int(r["route"].n_rows[2]) > 0


def test_hybrid_cap_zero_equals_plain_fused():
    """With no dense rows every row is served from TwELL: rows of ordinary
    weight equal the plain fused kernel bit for bit; the heavy rows (total
    non-zeros > max(2 C, 2 x mean), which the hybrid path cuts into tile
    ranges summed in a fixed order) agree within the bf16 tolerance."""
    w = W.workload(4, T=700)
    r = run_hybrid(w, 0, label="cap=0")
    y2 = torch.empty_like(r["y"])
    x, wu, wd = (dev(r["inp"][k + "_raw"], w.dtype) for k in ("x", "w_up_t", "w_down"))
    T.twell_ffn_fwd(r["desc"], x, r["act"], wu, wd, y2)
    torch.cuda.synchronize()
    tot = r["act"].count.cpu().numpy().clip(min=0).sum(axis=1)
    heavy = tot > max(2.0 * w.slots, 2.0 * np.float32(tot.sum() / w.T))
    assert heavy.any() and not heavy.all()
    light = torch.from_numpy(~heavy).cuda()
    assert torch.equal(r["y"][light].view(torch.int16), y2[light].view(torch.int16))
    yh, y2h = host64(r["y"])[heavy], host64(y2)[heavy]
    assert np.abs(yh - y2h).max() <= 1e-2 * np.abs(y2h).max()


def test_hybrid_all_rows_dense():
    w = W.workload(5, T=300, rho=0.3)   # every row overflows
    r = run_hybrid(w, 300, label="all dense")
    assert int(r["route"].n_rows[0]) == 0


def test_hybrid_fp32():
    import dataclasses
    w = dataclasses.replace(W.workload(1), slots=2)  # few slots: some rows go dense
    run_hybrid(w, 256, label="fp32 C=2")


def test_hybrid_full_size_sampled():
    w = W.workload(4)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(w.T - 256, w.T), rng.choice(w.T, 256, replace=False)]))
    run_hybrid(w, 1024, rows=rows, label="full c4")


def test_hybrid_lockstep_four_rows_per_wave_sampled():
    # d_model = 1024 at 16384 rows: the lockstep kernel holds 4 rows per wave, so
    # its row dealing ranks 512 rows per window of 8 workgroups
    w = W.workload(4, d_model=1024, d_ff=4096)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(w.T - 128, w.T), rng.choice(w.T, 256, replace=False)]))
    run_hybrid(w, 1024, rows=rows, label="lognormal d=1024")


def test_hybrid_wide_rows_lockstep_sampled():
    # d_model = 4096 at 4096 rows: the light rows take the 8-wave lockstep
    # kernel, dealt over windows of 8 workgroups by their totals
    w = W.workload(4, T=4096, d_model=4096, d_ff=11008)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(w.T - 128, w.T), rng.choice(w.T, 192, replace=False)]))
    run_hybrid(w, 256, rows=rows, label="lognormal d=4096")


def test_hybrid_wide_rows_per_token():
    # d_model = 4096 below 2048 rows: the light rows take the 8-wave per-token workgroups
    run_hybrid(W.workload(4, T=300, d_model=4096, d_ff=8192), 64, label="lognormal d=4096 T=300")


def test_hybrid_deterministic_lockstep():
    """A batch large enough for the lockstep fused kernel (whose chunk order
    depends on the workgroup), with heavy and dense rows: two calls give the
    same bits."""
    w = W.workload(4, T=2600)
    rows = np.arange(0, w.T, 13)
    r = run_hybrid(w, 128, rows=rows, label="determinism a")
    x, wg, wu, wd = (dev(r["inp"][k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
    ws = torch.empty(T.sizes(r["desc"], 128)["ws_hybrid"], dtype=torch.uint8, device="cuda")
    route2 = T.alloc_route(r["desc"], 128)
    y2 = poison_(torch.empty_like(r["y"]))
    T.twell_ffn_fwd_hybrid(r["desc"], x, wg, r["act"], wu, wd, y2, route2, ws)
    torch.cuda.synchronize()
    assert torch.equal(r["y"].view(torch.int16), y2.view(torch.int16))
