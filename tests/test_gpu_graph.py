"""The forward entry points under HIP graph capture.

The library launches kernels only (no allocation, memset, copy or host
synchronisation inside any entry point), so a caller can capture a forward
pass into a graph and replay it -- the use the allocation-free hybrid entry
point exists for.  Each test runs the entry points eagerly, captures the same
calls into a torch CUDA graph (on HIP, a hipGraph) writing separate output
buffers, then replays the graph several times with eager work in between
(the outputs are overwritten with a byte pattern before each replay) and
checks every replay bit for bit against the eager outputs.  Nothing but
library calls is recorded in the graphs.
"""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from _helpers import desc_for, dev, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _weights(w):
    inp = W.make_inputs(w)
    return inp, [dev(inp[k + "_raw"], w.dtype) for k in ("x", "w_gate_t", "w_up_t", "w_down")]


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _replay_and_check(g, outs, refs, label):
    for r in range(REPLAYS):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert _same(o, ref), f"{label}: replay {r}, output {i} differs from the eager result"


# 16 rows: small-batch kernels; 2100: one lockstep dispatch; 16384: two lockstep dispatches
@pytest.mark.parametrize("t_rows", [16, 2100, 16384])
def test_pack_and_fused_forward_replay_bitwise(t_rows):
    say(f"[gpu case] graph capture of twell_pack + twell_ffn_fwd, 2B shape, T={t_rows}")
    w = W.workload(3, T=t_rows)
    desc = desc_for(w)
    _, (x, wg, wu, wd) = _weights(w)
    act = T.alloc_act(desc)
    y = torch.empty((w.T, w.d_model), dtype=desc.torch_dtype, device="cuda")
    T.twell_pack(desc, x, wg, act)
    T.twell_ffn_fwd(desc, x, act, wu, wd, y)
    torch.cuda.synchronize()
    refs = [t.clone() for t in (*act, y)]

    act_g = T.alloc_act(desc)
    y_g = torch.empty_like(y)

    def fwd():
        T.twell_pack(desc, x, wg, act_g)
        T.twell_ffn_fwd(desc, x, act_g, wu, wd, y_g)

    g = _capture(fwd)
    _replay_and_check(g, [*act_g, y_g], refs, f"T={t_rows}")


@pytest.mark.parametrize("t_rows", [300, 2100])
def test_allocation_free_hybrid_forward_replay_bitwise(t_rows):
    say(f"[gpu case] graph capture of twell_pack + twell_ffn_fwd_hybrid_noalloc, training shape, T={t_rows}")
    w = W.workload(4, T=t_rows)
    desc = desc_for(w)
    _, (x, wg, wu, wd) = _weights(w)
    cap = 64
    act = T.alloc_act(desc)
    route = T.alloc_route(desc, cap)
    y = torch.empty((w.T, w.d_model), dtype=desc.torch_dtype, device="cuda")
    T.twell_pack(desc, x, wg, act)
    T.twell_ffn_fwd_hybrid_noalloc(desc, x, wg, act, wu, wd, y, route)
    torch.cuda.synchronize()
    n_rows = route.n_rows.cpu().tolist()
    assert n_rows[0] > 0 and n_rows[1] > 0, "the case should route rows both ways"
    refs = [y.clone(), route.n_rows.clone(), route.row_kind.clone(),
            route.ell_rows[:n_rows[0]].clone(), route.dense_rows[:min(n_rows[1], cap)].clone()]

    act_g = T.alloc_act(desc)
    route_g = T.alloc_route(desc, cap)
    y_g = torch.empty_like(y)

    def fwd():
        T.twell_pack(desc, x, wg, act_g)
        T.twell_ffn_fwd_hybrid_noalloc(desc, x, wg, act_g, wu, wd, y_g, route_g)

    g = _capture(fwd)
    for r in range(REPLAYS):
        for o in (y_g, route_g.ell_rows, route_g.dense_rows, route_g.row_kind, route_g.n_rows, *act_g):
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y_g, route_g.n_rows, route_g.row_kind, route_g.ell_rows[:n_rows[0]],
               route_g.dense_rows[:min(n_rows[1], cap)]]
        for i, (o, ref) in enumerate(zip(got, refs)):
            assert _same(o, ref), f"hybrid T={t_rows}: replay {r}, output {i} differs from the eager result"
    # and the eager result itself is the workspace entry point's
    ws = torch.empty(T.sizes(desc, cap)["ws_hybrid"], dtype=torch.uint8, device="cuda")
    y_ws = torch.empty_like(y)
    route_ws = T.alloc_route(desc, cap)
    T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y_ws, route_ws, ws)
    torch.cuda.synchronize()
    assert _same(y_ws, refs[0])
    assert np.array_equal(route_ws.n_rows.cpu().numpy(), np.asarray(n_rows))
