"""GPU parity of the classic ELL baseline (twell_pack_classic: dense gate GEMM
writing ReLU(g), then a conversion kernel) through the C ABI.

twell_pack is pinned bit-exactly to the oracle packer elsewhere.  Where both
paths run the same GEMM core (the 256-row tiles: every fp32 or T_n = 64 batch,
and bf16 T_n = 128 batches too large for one generation of the mid-size
kernel's workgroups) the classic path must produce
byte-identical TwELL planes and its dense ReLU(g) must equal the pack kernel's
own dense debug output.  Below that (bf16, T_n = 128) twell_pack runs the
small / mid-size kernel, which sums K in two groups: there each dense output
lies within the fp32-accumulation bound of the float64 ReLU(g), and each
path's planes are exactly the oracle packer applied to its own dense output."""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W
from oracle import twell_oracle as O
from _helpers import check_guards, desc_for, dev, guarded, guarded_act, host64, say

pytestmark = pytest.mark.gpu

CASES = [
    ("c1 fp32 T_n=64", W.workload(1)),
    ("c2 ragged T", W.workload(2, T=1000)),
    ("c3 shape T=300", W.workload(3, T=300)),
    ("rho 5% (overflow)", W.workload(5, T=300, rho=0.05)),
    ("C = T_n", W.workload(2, T=260, rho=0.3)),
    ("T=1", W.workload(2, T=1)),
    ("c3 full", W.workload(3)),
]


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_classic_equals_epilogue_pack(label, w):
    if label == "C = T_n":
        import dataclasses
        w = dataclasses.replace(w, slots=w.tile_n)
    say(f"[gpu case] classic {label} T={w.T} F={w.d_ff} C={w.slots} {w.dtype}")
    inp = W.make_inputs(w)
    desc = desc_for(w)
    x = dev(inp["x_raw"], w.dtype)
    wg = dev(inp["w_gate_t_raw"], w.dtype)
    a1, a2 = guarded_act(desc), guarded_act(desc)
    gate = guarded((desc.T, desc.d_ff), desc.torch_dtype)
    T.twell_pack(desc, x, wg, a1, gate_dbg=gate)
    ws = guarded((T.sizes(desc)["ws_pack_classic"],), torch.uint8)
    T.twell_pack_classic(desc, x, wg, a2, ws)
    torch.cuda.synchronize()
    check_guards(*a1, *a2, gate, ws)
    dense = ws[: desc.T * desc.d_ff * (2 if w.dtype == "bf16" else 4)].view(desc.torch_dtype).view(desc.T, desc.d_ff)
    # the small / mid-size gate kernel: up to 64 tokens, and blocks of 128 tokens while all its
    # workgroups run in one generation (d_ff/128 tiles x blocks <= CUs), up to 2048 tokens
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mid = desc.T <= 2048 and (desc.d_ff // 128) * ((desc.T + 127) // 128) <= cus
    same_core = not (w.dtype == "bf16" and desc.tile_n == 128 and (desc.T <= 64 or mid))
    if same_core:
        assert torch.equal(dense.view(torch.int16 if w.dtype == "bf16" else torch.int32),
                           gate.view(torch.int16 if w.dtype == "bf16" else torch.int32))
        for p1, p2, name in zip(a1, a2, ("count", "idx", "val")):
            b1 = p1.view(torch.uint8) if p1.dtype != torch.uint8 else p1
            b2 = p2.view(torch.uint8) if p2.dtype != torch.uint8 else p2
            assert torch.equal(b1, b2), name
    else:
        # each dense output within the fp32-accumulation bound of the float64 ReLU(g) (next to
        # zero one path may round a sum to a tiny value the other clamps to 0, so no relative test)
        d64, g64 = host64(dense), host64(gate)
        a_ref = O.ffn_forward(inp["x"], inp["w_gate_t"], inp["w_up_t"], inp["w_down"])["a"]
        bound = O.gate_error_bound(inp["x"], inp["w_gate_t"], w.dtype)
        for name, v in (("classic", d64), ("epilogue", g64)):
            assert np.all(np.abs(v - a_ref) <= bound), f"{name} dense ReLU(g) outside the accumulation bound"
        cnt, idx, val = O.twell_pack(g64, desc.tile_n, desc.slots)  # the pack kernel on its own output
        assert np.array_equal(a1.count.cpu().numpy(), cnt)
        assert np.array_equal(a1.idx.cpu().numpy(), idx)
        assert np.array_equal(host64(a1.val), val)
    if desc.T <= 1000:  # the classic path against the oracle packer on its own dense output
        cnt, idx, val = O.twell_pack(host64(dense), desc.tile_n, desc.slots)
        assert np.array_equal(a2.count.cpu().numpy(), cnt)
        assert np.array_equal(a2.idx.cpu().numpy(), idx)
        assert np.array_equal(host64(a2.val), val)
