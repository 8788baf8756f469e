"""GPU parity of the inference path (twell_pack, twell_ffn_fwd) and of the
library's dense FFN against the CPU oracle, called through the C ABI.

Checks per case:
  * gate: every stored activation ReLU(g) (the kernel's debug dense output)
    lies within the fp32-accumulation + storage-rounding bound of the oracle's
    float64 ReLU(g);
  * pack: the kernel's TwELL equals, bit for bit, the oracle packer applied to
    the kernel's own dense gate output, on every row (also at full size); the
    device stats equal the counts;
  * fused forward: y within tol * max|y_ref| of the oracle's TwELL forward on
    the kernel's TwELL (tol 1e-5 fp32, 1e-2 bf16), and of the oracle's dense
    FFN wherever no tile overflows;
  * dense FFN: y within the same tolerance of the oracle's dense FFN;
  * every output buffer sits between canary regions that must stay untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from oracle import twell_oracle as O
from _helpers import (assert_rows_written, check_guards, desc_for, dev, guarded, guarded_act, host64, record, say,
                      within)

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def _run_pack_fwd(w, desc, inp, dbg=True):
    x = dev(inp["x_raw"], w.dtype)
    wg = dev(inp["w_gate_t_raw"], w.dtype)
    wu = dev(inp["w_up_t_raw"], w.dtype)
    wd = dev(inp["w_down_raw"], w.dtype)
    act = guarded_act(desc)
    stats = guarded((2,), torch.int64)
    stats.zero_()
    gate = guarded((desc.T, desc.d_ff), desc.torch_dtype) if dbg else None
    y = guarded((desc.T, desc.d_model), desc.torch_dtype)
    T.twell_pack(desc, x, wg, act, stats=stats, gate_dbg=gate)
    T.twell_ffn_fwd(desc, x, act, wu, wd, y)
    torch.cuda.synchronize()
    check_guards(*act, stats, y, *([gate] if dbg else []))
    assert_rows_written(y, "y")
    return dict(x=x, wg=wg, wu=wu, wd=wd, act=act, stats=stats, gate=gate, y=y)


def _check_case(w, rows=None, label=""):
    """Run pack + fused forward on workload w and check every output against the oracle.
    The TwELL planes are compared byte for byte on every row; rows: host row
    sample for the float64 checks of the gate and of y (None = all rows)."""
    say(f"[gpu case] {label} {w.name} T={w.T} d={w.d_model} F={w.d_ff} Tn={w.tile_n} C={w.slots} {w.dtype}")
    inp = W.make_inputs(w)
    desc = desc_for(w)
    r = _run_pack_fwd(w, desc, inp)
    count = r["act"].count.cpu().numpy()
    idx = r["act"].idx.cpu().numpy()
    val = host64(r["act"].val)
    gate = host64(r["gate"])
    stats = r["stats"].cpu().numpy()
    y = host64(r["y"])
    sel = np.arange(w.T) if rows is None else np.asarray(rows)

    # pack: bit-exact against the oracle packer on the kernel's own gate output, all rows
    oc, oi, ov = O.twell_pack(gate, w.tile_n, w.slots)
    np.testing.assert_array_equal(count, oc)
    np.testing.assert_array_equal(idx, oi)
    np.testing.assert_array_equal(val, ov)
    del oc, oi, ov
    assert stats[1] == int(count.astype(np.int64).sum())
    assert stats[0] == int((count > w.slots).sum())

    # gate values within the accumulation bound
    xs = inp["x"][sel]
    f = O.ffn_forward(xs, inp["w_gate_t"], inp["w_up_t"], inp["w_down"])
    bound = O.gate_error_bound(xs, inp["w_gate_t"], w.dtype)
    err = np.abs(gate[sel] - f["a"])
    assert np.all(err <= bound), f"gate error {err.max()} > bound at {np.unravel_index(np.argmax(err - bound), err.shape)}"

    # fused forward against the oracle's TwELL forward on the kernel's TwELL
    y_tw = O.twell_forward(xs, count[sel], idx[sel], val[sel], w.tile_n, inp["w_up_t"], inp["w_down"])
    tol = TOL[w.dtype]
    scale = max(np.abs(y_tw).max(), 1e-30)
    within(y[sel], y_tw, tol, f"{label} {w.name} T={w.T}: y vs oracle TwELL forward")
    if w.dtype == "bf16":
        # how much of that is the kernel's rounding of h to bf16 before the W_down product (the
        # precision a dense bf16 FFN stores h in): the same product with only that rounding applied
        h = O.twell_unpack(count[sel], idx[sel], val[sel], w.tile_n) * (xs @ np.asarray(inp["w_up_t"], np.float64).T)
        y_h = O.round_to_storage(h, "bf16") @ np.asarray(inp["w_down"], np.float64)
        record(f"{label} {w.name} T={w.T}: y moved by rounding h to bf16 alone", float(np.abs(y_h - y_tw).max() / scale))
    # and end to end against the dense FFN on rows with no overflowing tile
    ok = ~(count[sel] > w.slots).any(axis=1)
    if ok.any():
        within(y[sel][ok], f["y"][ok], tol, f"{label} {w.name} T={w.T}: y vs oracle dense FFN")
    density = count.astype(np.int64).sum() / (w.T * w.d_ff)
    say(f"   ok: density {density:.5f}, overflow tiles {stats[0]}, max|y| {scale:.3g}")
    return r, inp


CASES = [
    ("c1 full", W.workload(1)),
    ("c1 ragged T", W.workload(1, T=77)),
    ("c2 ragged T", W.workload(2, T=1000)),
    ("c3 shape T=600", W.workload(3, T=600)),
    ("c5 rho 5% (overflow)", W.workload(5, T=300, rho=0.05)),
    ("c5 rho 0.1%", W.workload(5, T=300, rho=0.001)),
    ("c5 rho 1%", W.workload(5, T=300, rho=0.01)),
    ("c5 rho 2%", W.workload(5, T=300, rho=0.02)),
    ("c5 T=16", W.workload(5, T=16)),
    ("T=1", W.workload(2, T=1)),
    # the small-batch gate kernel stages 16, 32 or 64 token rows by batch size
    ("small batch T=11", W.workload(3, T=11)),
    ("small batch T=31", W.workload(3, T=31)),
    ("small batch T=57 rho 2%", W.workload(5, T=57, rho=0.02)),
    # up to 512 tokens the same kernel runs blocks of 128 tokens (a second grid dimension)
    ("mid batch T=129", W.workload(3, T=129)),
    ("mid batch T=512 rho 2%", W.workload(5, T=512, rho=0.02)),
    ("c4 lognormal tail", W.workload(4, T=520)),
    ("c3 8-way neuron shard F=1024", W.workload(3, T=600, d_ff=1024)),
    ("wide d_ff=16384", W.workload(4, T=300, d_model=512, d_ff=16384)),
    # below 2048 rows, bf16 rows wider than 2048 take the 8-wave per-token workgroups
    ("wide rows d=4096 T=16", W.workload(3, T=16, d_model=4096, d_ff=11008)),
    ("wide rows d=3072 T=300", W.workload(5, T=300, d_model=3072, d_ff=8192, rho=0.02)),
    # batches of 2048+ tokens take the lockstep fused kernel (smaller ones the per-token kernel)
    ("lockstep ragged T=2049", W.workload(2, T=2049)),
    ("lockstep C=T_n T=2080", dataclasses.replace(W.workload(2, T=2080, rho=0.3), slots=128)),
    ("lockstep c4 tail T=2100", W.workload(4, T=2100)),
    ("lockstep wide d_ff=16384", W.workload(3, T=2048, d_model=512, d_ff=16384)),
]


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_pack_and_fused_forward(label, w):
    _check_case(w, label=label)


def test_bf16_tile64_and_full_capacity_slots():
    # tile_n = 64 in bf16, and C = tile_n (no overflow possible) at high density,
    # which also drives the fused kernel through several chunks of tiles
    import dataclasses
    w = dataclasses.replace(W.workload(2, T=130, rho=0.3), tile_n=64, slots=64)
    _check_case(w, label="tile64 C=64 rho=30%")
    w = dataclasses.replace(W.workload(2, T=70, rho=0.5), tile_n=128, slots=128)
    _check_case(w, label="C=128 rho=50%")


def test_all_gates_off():
    w = W.workload(2, T=64, rho=1e-9)  # column-0 offset ~ 6 sigma: no gate fires
    r, _ = _check_case(w, label="all off")
    assert int(r["act"].count.sum()) == 0
    assert torch.all(r["y"] == 0)
    assert torch.all(r["act"].idx == 0) and torch.all(r["act"].val == 0)


def test_pack_without_debug_output_is_identical_and_deterministic():
    w = W.workload(3, T=700)
    inp = W.make_inputs(w)
    desc = desc_for(w)
    say("[gpu case] dbg vs no-dbg determinism")
    a = _run_pack_fwd(w, desc, inp, dbg=True)
    b = _run_pack_fwd(w, desc, inp, dbg=False)
    c = _run_pack_fwd(w, desc, inp, dbg=False)
    for k in range(3):
        assert torch.equal(a["act"][k].view(torch.uint8), b["act"][k].view(torch.uint8))
        assert torch.equal(b["act"][k].view(torch.uint8), c["act"][k].view(torch.uint8))
    assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))
    assert torch.equal(b["y"].view(torch.int16), c["y"].view(torch.int16))


def test_empty_batch():
    w = W.workload(2)
    desc = desc_for(w, T=0)
    e = torch.empty(0, device="cuda", dtype=torch.bfloat16)
    act = T.alloc_act(desc)
    T.twell_pack(desc, e, torch.empty((w.d_ff, w.d_model), device="cuda", dtype=torch.bfloat16), act)
    torch.cuda.synchronize()


DENSE_CASES = [
    ("c1", W.workload(1)),
    ("c2 ragged", W.workload(2, T=700)),
    ("c3 shape", W.workload(3, T=300)),
    ("rho 5%", W.workload(5, T=260, rho=0.05)),
    ("c3 8-way neuron shard F=1024", W.workload(3, T=600, d_ff=1024)),
]


@pytest.mark.parametrize("label,w", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_ffn(label, w):
    say(f"[gpu case] dense {label} T={w.T}")
    inp = W.make_inputs(w)
    desc = desc_for(w)
    x, wg, wu, wd = (dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
    y = guarded((w.T, w.d_model), desc.torch_dtype)
    ws = guarded((T.sizes(desc)["ws_dense_fwd"],), torch.uint8)
    T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    check_guards(y, ws)
    yr = O.ffn_forward(inp["x"], inp["w_gate_t"], inp["w_up_t"], inp["w_down"])["y"]
    within(host64(y), yr, TOL[w.dtype], f"dense {label} T={w.T}: y vs oracle dense FFN")


# ----------------------------------------------------------------------------- full size
def _sample_rows(T_, seed=0, n_rand=192):
    rng = np.random.default_rng(seed)
    rows = set(range(0, min(T_, 256))) | set(range(max(0, T_ - 256), T_))
    rows |= set(rng.choice(T_, size=min(n_rand, T_), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_sampled_rows(cfg):
    """Full workload sizes, the launch configuration the benchmark times: TwELL
    byte for byte on all rows, float64 checks of the gate and y on sampled rows
    (the first and last 256 rows plus 192 random ones)."""
    w = W.workload(cfg)
    r, _ = _check_case(w, rows=_sample_rows(w.T, cfg), label=f"full c{cfg}")
    # two generations of lockstep workgroups at c3: a second call gives the same bits
    y2 = guarded(tuple(r["y"].shape), r["y"].dtype)
    T.twell_ffn_fwd(desc_for(w), r["x"], r["act"], r["wu"], r["wd"], y2)
    torch.cuda.synchronize()
    check_guards(y2)
    assert torch.equal(r["y"].view(torch.int16), y2.view(torch.int16))


def test_lockstep_three_generations_sampled():
    """24 608 tokens (d_model = 512): 769 lockstep workgroups of 32 rows, i.e.
    three launches of one generation each on 256 CUs and a ragged fourth of one
    workgroup, so the per-generation launch offsets and the rotation shift of
    every later generation run; rows around each generation boundary are
    checked."""
    w = W.workload(3, T=24608, d_model=512)
    rows = set(_sample_rows(w.T, 11).tolist())
    for b in (8192, 16384, 24576):
        rows |= set(range(b - 64, min(b + 64, w.T)))
    _check_case(w, rows=np.array(sorted(rows)), label="three generations")


@pytest.mark.parametrize("T_,d,F", [(4096, 4096, 11008), (8192, 3072, 8192)], ids=["d4096 one generation",
                                                                                "d3072 two generations"])
def test_lockstep_wide_rows_sampled(T_, d, F):
    """bf16 rows wider than 2048 from 4096 tokens on take the 8-wave lockstep
    kernel (two rows per wave, chunks of at most 2 tiles at d_model = 4096):
    TwELL byte for byte on all rows, the gate and y on sampled rows, and a
    second call gives the same bits."""
    w = W.workload(3, T=T_, d_model=d, d_ff=F)
    r, _ = _check_case(w, rows=_sample_rows(w.T, d), label="wide lockstep")
    y2 = guarded(tuple(r["y"].shape), r["y"].dtype)
    T.twell_ffn_fwd(desc_for(w), r["x"], r["act"], r["wu"], r["wd"], y2)
    torch.cuda.synchronize()
    check_guards(y2)
    assert torch.equal(r["y"].view(torch.int16), y2.view(torch.int16))


def test_dense_ffn_full_size_sampled():
    """The dense FFN in the configuration the benchmark times (2B-class shape,
    T=16384), checked on sampled rows against the float64 dense FFN."""
    w = W.workload(3)
    say(f"[gpu case] dense full c3 T={w.T}")
    inp = W.make_inputs(w)
    desc = desc_for(w)
    x, wg, wu, wd = (dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
    y = guarded((w.T, w.d_model), desc.torch_dtype)
    ws = guarded((T.sizes(desc)["ws_dense_fwd"],), torch.uint8)
    T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    check_guards(y, ws)
    rows = _sample_rows(w.T, 7)
    yr = O.ffn_forward(inp["x"][rows], inp["w_gate_t"], inp["w_up_t"], inp["w_down"])["y"]
    within(host64(y)[rows], yr, TOL[w.dtype], f"dense full T={w.T}: y vs oracle dense FFN (sampled rows)")
