"""The allocation-free hybrid forward (twell_ffn_fwd_hybrid_noalloc, whose
workspace is the library's static device scratch) against the workspace entry
point twell_ffn_fwd_hybrid, through the C ABI: same y bits and same route
outputs, on two calls in a row, the second with a smaller input (so the
scratch holds the first call's contents when the second starts)."""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from _helpers import check_guards, desc_for, dev, guarded, guarded_act, guarded_route, say

pytestmark = pytest.mark.gpu


def _inputs(w):
    inp = W.make_inputs(w)
    return tuple(dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down"))


def test_noalloc_hybrid_equals_workspace_entry_point_on_two_calls():
    # first a lockstep-sized batch with heavy and dense rows, then a smaller one
    for T_, cap in ((2600, 128), (700, 64)):
        w = W.workload(4, T=T_)
        say(f"[gpu case] noalloc hybrid T={T_} cap={cap}")
        desc = desc_for(w)
        assert T.sizes(desc, cap)["ws_hybrid"] <= T.NOALLOC_SCRATCH_BYTES
        x, wg, wu, wd = _inputs(w)
        act = guarded_act(desc)
        T.twell_pack(desc, x, wg, act)
        r1, r2 = guarded_route(desc, cap), guarded_route(desc, cap)
        y1 = guarded((w.T, w.d_model), desc.torch_dtype)
        y2 = guarded((w.T, w.d_model), desc.torch_dtype)
        ws = guarded((T.sizes(desc, cap)["ws_hybrid"],), torch.uint8)
        T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y1, r1, ws)
        T.twell_ffn_fwd_hybrid_noalloc(desc, x, wg, act, wu, wd, y2, r2)
        torch.cuda.synchronize()
        check_guards(*act, *r1, *r2, y1, y2, ws)
        n = r1.n_rows.cpu().numpy()
        assert n[1] > 0 and n[0] > 0  # both the dense fallback and the TwELL rows ran
        assert np.array_equal(n, r2.n_rows.cpu().numpy())
        assert torch.equal(r1.ell_rows[:n[0]], r2.ell_rows[:n[0]])
        assert torch.equal(r1.dense_rows[:n[1]], r2.dense_rows[:n[1]])
        assert torch.equal(r1.row_kind, r2.row_kind)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        say(f"   ok: n_ell={n[0]} n_dense={n[1]}")


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    w = W.workload(4)
    desc = desc_for(w)
    cap = 1024
    assert T.sizes(desc, cap)["ws_hybrid"] > T.NOALLOC_SCRATCH_BYTES
    x, wg, wu, wd = (torch.empty((n, w.d_model), dtype=torch.bfloat16, device="cuda") for n in (w.T, w.d_ff, w.d_ff,
                                                                                                  w.d_ff))
    act = T.alloc_act(desc)
    route = T.alloc_route(desc, cap)
    y = torch.empty((w.T, w.d_model), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(T.TwellError) as e:
        T.twell_ffn_fwd_hybrid_noalloc(desc, x, wg, act, wu, wd, y, route)
    assert e.value.code == T.TWELL_ESCRATCH
