"""GPU pin of the value the gate kernels store: the storage rounding of ReLU(g)
(TwELL page, section on what TwELL does differently from classic ELL: the
non-zeros of the gate output are packed in the matmul's epilogue), bit for bit.

The float32-accumulation bound of the other forward tests is wider than a bf16
ulp wherever the accumulation term dominates, so a kernel that truncated
instead of rounding to nearest, or broke ties the wrong way, could pass them.
Here the inputs make the gate exact in float32 whatever the summation order:
x[t] = (1, s_t, 0, ...) with s_t in {1/4, 1, 2, 8}, and W_gate^T[j] = (a_j, b_j,
0, ...) with a_j a bf16 value in [0.5, 4) and b_j = k_j * 2^(e_j - 16), k_j < 256
an integer and 2^e_j the binade of a_j.  Then g = a_j + s_t * b_j spans at most
21 bits, every partial sum is exact, and ReLU(g) in bf16 is decided by its bits
below the 8th: below half an ulp, exactly half (ties, both parities of a_j's
last bit), above half, and carries into the next binade (a_j = 255/128 * 2^e_j).
Inactive neurons have g = -1.  Every stored value, and the debug copy of the
dense gate, must equal the oracle's round-to-nearest-even of the exact float64
gate; float32 storage must hold g itself.  Cases cover the 256-row epilogue
(bf16 C = 16 and a C = 12 format), the 64-wide tile kernel, the small-batch
kernel (T <= 64), float32, and the classic dense-then-convert construction.
"""
import numpy as np
import pytest
import torch

from activation_sparse_feedforward_amd import twell as T
from oracle import twell_oracle as O
from _helpers import check_guards, guarded, guarded_act, host64, say

pytestmark = pytest.mark.gpu

D_MODEL, D_FF = 512, 1024


def _bf16_tensor(v: np.ndarray) -> torch.Tensor:
    """float64 values that are exact in bf16 -> a GPU bf16 tensor with those bits."""
    f = np.ascontiguousarray(v, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "input value not representable in bf16"
    return torch.from_numpy((bits >> 16).astype(np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def _exact_inputs(t_rows: int, tile_n: int, slots: int, seed: int):
    """x [T x D_MODEL] and W_gate^T [D_FF x D_MODEL] (float64, exact in bf16)
    whose gate is exact in float32 and exercises every rounding case; every
    tile holds min(12, slots) active neurons, so none overflows."""
    n_act = min(12, slots)
    rng = np.random.default_rng(seed)
    s = np.array([2.0, 8.0, 1.0, 0.25])[np.arange(t_rows) % 4]   # every batch has rows with s = 2
    x = np.zeros((t_rows, D_MODEL))
    x[:, 0] = 1.0
    x[:, 1] = s
    w = np.zeros((D_FF, D_MODEL))
    w[:, 0] = -1.0                                   # inactive: g = -1
    n_t = D_FF // tile_n
    for b in range(n_t):
        cols = b * tile_n + rng.choice(tile_n, size=n_act, replace=False)
        e = rng.integers(-1, 2, size=n_act)               # binade of a: [2^e, 2^(e+1))
        m = rng.integers(0, 128, size=n_act)              # a = (128 + m) / 128 * 2^e
        k = rng.integers(0, 256, size=n_act)              # b = k * 2^(e - 16)
        # forced cases, seen by the rows with s = 2 (s * b = k * 2^(e - 15); half an ulp of a is
        # 2^(e - 8), i.e. k = 128): a = 255/128 * 2^e with a tie, above half and below half (the
        # first two carry into the next binade), then a tie on an even and on an odd last bit of a
        m[:6] = [127, 127, 127, 0, 1, 2]
        k[:6] = [128, 192, 64, 128, 128, 192]
        w[cols, 0] = (128 + m) / 128.0 * np.exp2(e)
        w[cols, 1] = k * np.exp2(e - 16.0)
    return x, w


def _expected(x, w, tile_n, slots, dtype):
    g, a = O.gate_forward(x, w)
    assert np.all(np.abs(g) < 2.0 ** 4)
    a_s = O.round_to_storage(a, dtype)
    return a_s, O.twell_pack(a_s, tile_n, slots)


CASES = [
    # (T, tile_n, slots, dtype, path)
    (2100, 128, 16, "bf16", "epilogue"),     # 256 x 256 tiles, row-staged epilogue, ragged last tile
    (600, 128, 12, "bf16", "epilogue"),      # 256 x 256 tiles, register epilogue (C != 16)
    (300, 64, 8, "bf16", "epilogue"),        # 64-wide tiles
    (16, 128, 16, "bf16", "epilogue"),       # small-batch kernel
    (300, 64, 8, "fp32", "epilogue"),
    (2100, 128, 16, "bf16", "classic"),      # dense ReLU(g) write-back + conversion
]


@pytest.mark.parametrize("t_rows,tile_n,slots,dtype,path", CASES,
                         ids=[f"T{c[0]}_Tn{c[1]}_C{c[2]}_{c[3]}_{c[4]}" for c in CASES])
def test_stored_activation_is_the_rounded_exact_gate(t_rows, tile_n, slots, dtype, path):
    say(f"[gpu case] exact-gate rounding T={t_rows} Tn={tile_n} C={slots} {dtype} {path}")
    x, w = _exact_inputs(t_rows, tile_n, slots, seed=t_rows + tile_n + slots)
    a_s, (oc, oi, ov) = _expected(x, w, tile_n, slots, dtype)
    # the cases the docstring promises are all present among the active values
    if dtype == "bf16":
        g = O.gate_forward(x, w)[0]
        live = g > 0
        _, ex = np.frexp(np.where(live, g, 1.0))         # g in [2^(ex-1), 2^ex)
        step = np.exp2(ex - 8.0)                          # bf16 ulp of g
        rem = np.where(live, np.mod(g, step) / step, -1.0)
        assert np.any(rem == 0.5) and np.any((rem > 0) & (rem < 0.5)) and np.any(rem > 0.5)
        assert np.any(live & (a_s >= np.exp2(ex)))        # rounded up into the next binade

    desc = T.Desc(t_rows, D_MODEL, D_FF, tile_n, slots, dtype)
    if dtype == "bf16":
        xd, wd = _bf16_tensor(x), _bf16_tensor(w)
    else:
        xd = torch.from_numpy(x.astype(np.float32)).cuda()
        wd = torch.from_numpy(w.astype(np.float32)).cuda()
    act = guarded_act(desc)
    if path == "classic":
        ws = guarded((T.sizes(desc)["ws_pack_classic"],), torch.uint8)
        T.twell_pack_classic(desc, xd, wd, act, ws)
        torch.cuda.synchronize()
        check_guards(*act, ws)
    else:
        gate = guarded((t_rows, D_FF), desc.torch_dtype)
        stats = guarded((2,), torch.int64)
        stats.zero_()
        T.twell_pack(desc, xd, wd, act, stats=stats, gate_dbg=gate)
        torch.cuda.synchronize()
        check_guards(*act, stats, gate)
        np.testing.assert_array_equal(host64(gate), a_s)
        assert int(stats[0]) == 0 and int(stats[1]) == int((a_s != 0).sum())
    np.testing.assert_array_equal(act.count.cpu().numpy(), oc)
    np.testing.assert_array_equal(act.idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(host64(act.val), ov)
