"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (a hand-worked fixture, a closed form, an invariant, brute force on
tiny inputs, or central finite differences), so that a dropped term, a wrong
sign or index, or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import twell_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- pack
def test_pack_handworked_fixture():
    with open(os.path.join(GOLDEN, "twell_pack_handworked.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], dtype=np.float64)
    count, idx, val = O.twell_pack(A, g["tile_n"], g["slots"])
    np.testing.assert_array_equal(count, np.array(g["count"]))
    np.testing.assert_array_equal(idx, np.array(g["idx"]))
    np.testing.assert_array_equal(val, np.array(g["val"], dtype=np.float64))
    np.testing.assert_array_equal(O.twell_unpack(count, idx, val, g["tile_n"]), np.array(g["unpacked"]))
    dense, ell, dns = O.route(count, g["slots"])
    np.testing.assert_array_equal(ell, g["ell_rows"])
    np.testing.assert_array_equal(dns, g["dense_rows"])
    assert dense.tolist() == [r in g["dense_rows"] for r in range(A.shape[0])]


def _brute_pack(A, tile_n, C):
    """Pure-Python loops straight from the definition (tiny inputs only)."""
    T, F = A.shape
    n_t = F // tile_n
    count = np.zeros((T, n_t), np.int64)
    idx = np.zeros((T, n_t, C), np.int64)
    val = np.zeros((T, n_t, C))
    for t in range(T):
        for b in range(n_t):
            s = 0
            for c in range(tile_n):
                v = A[t, b * tile_n + c]
                if v != 0.0:
                    if s < C:
                        idx[t, b, s] = c
                        val[t, b, s] = v
                    s += 1
            count[t, b] = s
    return count, idx, val


def _adversarial_tiles(tile_n, C, rng):
    """One row per adversarial tile pattern, with positive values."""
    pats = []
    pats.append(np.zeros(tile_n))                                   # empty
    pats.append(np.ones(tile_n))                                    # full
    for k in (C - 1, C, C + 1):                                     # around capacity
        p = np.zeros(tile_n)
        p[rng.choice(tile_n, size=min(k, tile_n), replace=False)] = 1
        pats.append(p)
    p = np.zeros(tile_n); p[0] = 1; pats.append(p)                  # first column only
    p = np.zeros(tile_n); p[-1] = 1; pats.append(p)                 # last column only
    p = np.zeros(tile_n); p[::2] = 1; pats.append(p)                # alternating
    p = np.zeros(tile_n); p[1::2] = 1; pats.append(p)
    p = np.zeros(tile_n); p[-C:] = 1; pats.append(p)                # last C columns
    out = []
    for p in pats:
        out.append(p * rng.uniform(0.1, 4.0, tile_n))
    return out


@pytest.mark.parametrize("tile_n,C", [(8, 3), (64, 8), (128, 16), (128, 128), (64, 64)])
def test_pack_brute_force_adversarial(tile_n, C):
    rng = np.random.default_rng(100 + tile_n + C)
    pats = _adversarial_tiles(tile_n, C, rng)
    # every pattern in every tile position of a 3-tile row, plus random rows
    rows = []
    for p in pats:
        for pos in range(3):
            r = np.zeros(3 * tile_n)
            r[pos * tile_n:(pos + 1) * tile_n] = p
            rows.append(r)
    rnd = rng.uniform(0.1, 2.0, (12, 3 * tile_n)) * (rng.random((12, 3 * tile_n)) < 0.08)
    A = np.vstack(rows + list(rnd))
    count, idx, val = O.twell_pack(A, tile_n, C)
    bc, bi, bv = _brute_pack(A, tile_n, C)
    np.testing.assert_array_equal(count, bc)
    np.testing.assert_array_equal(idx, bi)
    np.testing.assert_array_equal(val, bv)
    # counts sum to nnz(A), always (count keeps the true count)
    assert int(count.sum()) == int(np.count_nonzero(A))


@pytest.mark.parametrize("seed", range(4))
def test_pack_roundtrip_exact(seed):
    rng = np.random.default_rng(seed)
    T, tile_n = 37, 64
    A = rng.standard_normal((T, 4 * tile_n))
    A = np.where(rng.random(A.shape) < 0.05, np.abs(A), 0.0)
    A = O.round_to_storage(A, "bf16")
    # at C = T_n nothing can overflow: exact inverse
    c, i, v = O.twell_pack(A, tile_n, tile_n)
    np.testing.assert_array_equal(O.twell_unpack(c, i, v, tile_n), A)
    # at small C: exact whenever no tile overflows
    c, i, v = O.twell_pack(A, tile_n, 8)
    if (c <= 8).all():
        np.testing.assert_array_equal(O.twell_unpack(c, i, v, tile_n), A)
    assert int(c.sum()) == int(np.count_nonzero(A))


def test_pack_uses_storage_nonzero():
    # a positive value that rounds to zero in bf16 takes no slot; -0.0 is zero
    A = np.zeros((1, 8))
    A[0, 1] = 2.0 ** -140          # far below half the smallest bf16 subnormal step
    A[0, 2] = -0.0
    A[0, 3] = 1.0
    As = O.round_to_storage(A, "bf16")
    c, i, v = O.twell_pack(As, 8, 4)
    assert c.tolist() == [[1]] and i[0, 0, 0] == 3 and v[0, 0, 0] == 1.0


def test_round_bf16_against_bit_rounding():
    # the oracle's float64 -> bf16 rounding agrees with integer round-to-nearest-even
    # on the float32 bit pattern for values exactly representable in float32
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # ties: construct exact halfway cases
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    u = a.view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    expect = r.astype(np.uint32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.round_to_storage(a, "bf16"), expect)


def test_round_bf16_hand_worked_cases():
    # bf16 keeps 8 significant bits, so in [1, 2) the step is 2^-7 and half a step 2^-8
    cases = [
        (1 + 2.0 ** -9, 1.0),                          # below half a step: down
        (1 + 2.0 ** -8, 1.0),                          # tie, 1.0 has an even last bit: stays
        (1 + 2.0 ** -7 + 2.0 ** -8, 1 + 2.0 ** -6),    # tie, 1 + 2^-7 has an odd last bit: up to even
        (1 + 2.0 ** -8 + 2.0 ** -12, 1 + 2.0 ** -7),   # above half: up
        (2 - 2.0 ** -8, 2.0),                          # tie at the top of the binade: carries to 2
        (3 * 2.0 ** -10 + 2.0 ** -19, 3 * 2.0 ** -10), # binade [2^-9, 2^-8), step 2^-16: below half
        (0.0, 0.0),
    ]
    got = O.round_to_storage(np.array([c[0] for c in cases]), "bf16")
    np.testing.assert_array_equal(got, [c[1] for c in cases])


# ----------------------------------------------------------------------------- forward
def _brute_ffn(x, wg, wu, wd):
    T, d = x.shape
    F = wg.shape[0]
    y = np.zeros((T, wd.shape[1]))
    for t in range(T):
        for j in range(F):
            g = sum(x[t, k] * wg[j, k] for k in range(d))
            u = sum(x[t, k] * wu[j, k] for k in range(d))
            a = g if g > 0 else 0.0
            for k in range(wd.shape[1]):
                y[t, k] += a * u * wd[j, k]
    return y


def test_forward_brute_force_nonsquare():
    rng = np.random.default_rng(11)
    T, d, F = 3, 5, 7
    x = rng.standard_normal((T, d))
    wg, wu, wd = rng.standard_normal((F, d)), rng.standard_normal((F, d)), rng.standard_normal((F, d))
    y = O.ffn_forward(x, wg, wu, wd)["y"]
    np.testing.assert_allclose(y, _brute_ffn(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_forward_all_gates_off_gives_zero():
    rng = np.random.default_rng(12)
    T, d, F = 16, 32, 64
    x = rng.standard_normal((T, d)) * 0.1
    x[:, 0] = 1.0
    wg = rng.standard_normal((F, d)) * 0.1
    wg[:, 0] = -100.0
    wu, wd = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    y = O.ffn_forward(x, wg, wu, wd)["y"]
    assert np.all(y == 0.0)


def test_forward_identity_closed_form():
    rng = np.random.default_rng(13)
    n = 64
    x = rng.standard_normal((9, n))
    I = np.eye(n)
    y = O.ffn_forward(x, I, I, I)["y"]
    np.testing.assert_array_equal(y, np.where(x > 0, x * x, 0.0))


def test_forward_single_active_neuron():
    rng = np.random.default_rng(14)
    T, d, F, j = 4, 8, 6, 3
    x = rng.standard_normal((T, d))
    x[:, 0] = 1.0
    wg = rng.standard_normal((F, d)) * 0.01
    wg[:, 0] = -10.0
    wg[j, 0] = 10.0
    wu, wd = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    f = O.ffn_forward(x, wg, wu, wd)
    a = x @ wg[j]
    u = x @ wu[j]
    np.testing.assert_allclose(f["y"], (a * u)[:, None] * wd[j][None, :], rtol=1e-14, atol=0)
    assert np.count_nonzero(f["a"]) == T


def test_sparse_equals_dense_and_per_slot_loop():
    """TwELL forward (oracle's own pack, C = T_n) equals the dense FFN fed the
    same storage-rounded activations, and equals a per-slot loop."""
    rng = np.random.default_rng(15)
    T, d, F, tile_n = 6, 16, 64, 16
    x = rng.standard_normal((T, d))
    x[:, 0] = 1.0
    wg = rng.standard_normal((F, d)) / 4
    wg[:, 0] = -0.6
    wu, wd = rng.standard_normal((F, d)) / 4, rng.standard_normal((F, d)) / 8
    f = O.ffn_forward(x, wg, wu, wd)
    a_s = O.round_to_storage(f["a"], "bf16")
    c, i, v = O.twell_pack(a_s, tile_n, tile_n)
    y_tw = O.twell_forward(x, c, i, v, tile_n, wu, wd)
    y_dense_rounded = (a_s * f["u"]) @ wd
    np.testing.assert_array_equal(y_tw, y_dense_rounded)
    y_loop = np.zeros_like(y_tw)
    for t in range(T):
        for b in range(F // tile_n):
            for s in range(min(c[t, b], tile_n)):
                j = b * tile_n + int(i[t, b, s])
                u = float(np.dot(x[t], wu[j]))
                y_loop[t] += v[t, b, s] * u * wd[j]
    np.testing.assert_allclose(y_tw, y_loop, rtol=1e-12, atol=1e-13)
    # and against the unrounded dense FFN within bf16 storage rounding
    assert np.max(np.abs(y_tw - f["y"])) <= 2.0 ** -8 * np.max(np.abs(f["a"] * f["u"])) * F * np.abs(wd).max()


def test_overflow_truncates_to_first_slots():
    rng = np.random.default_rng(16)
    T, d, F, tile_n, C = 5, 8, 16, 8, 2
    x = rng.standard_normal((T, d))
    a = np.abs(rng.standard_normal((T, F))) * (rng.random((T, F)) < 0.5)
    c, i, v = O.twell_pack(a, tile_n, C)
    kept = np.zeros_like(a)
    for t in range(T):
        for b in range(F // tile_n):
            nzc = [k for k in range(tile_n) if a[t, b * tile_n + k] != 0][:C]
            for k in nzc:
                kept[t, b * tile_n + k] = a[t, b * tile_n + k]
    wu, wd = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    y = O.twell_forward(x, c, i, v, tile_n, wu, wd)
    np.testing.assert_allclose(y, (kept * (x @ wu.T)) @ wd, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- hybrid
def test_route_brute_force():
    rng = np.random.default_rng(17)
    count = rng.integers(0, 20, (300, 6))
    dense, ell, dns = O.route(count, 16)
    exp_dense = [any(count[t, b] > 16 for b in range(6)) for t in range(300)]
    assert dense.tolist() == exp_dense
    assert ell.tolist() == [t for t in range(300) if not exp_dense[t]]
    assert dns.tolist() == [t for t in range(300) if exp_dense[t]]
    # degenerate: C = 0 sends every row with any non-zero dense; C = tile_n sends none
    d0, _, _ = O.route(count, 0)
    assert d0.tolist() == [bool((count[t] > 0).any()) for t in range(300)]
    dN, ellN, _ = O.route(count, 128)
    assert not dN.any() and ellN.size == 300


def test_hybrid_dense_rows_equal_ell_at_full_capacity():
    rng = np.random.default_rng(18)
    T, d, F, tile_n, C = 48, 16, 64, 16, 3
    x = rng.standard_normal((T, d))
    x[:, 0] = 1.0
    wg = rng.standard_normal((F, d)) / 4
    wg[:, 0] = -1.4
    wu, wd = rng.standard_normal((F, d)) / 4, rng.standard_normal((F, d)) / 8
    f = O.ffn_forward(x, wg, wu, wd)
    a_s = f["a"]  # float64 storage: the comparison below is exact
    c, i, v = O.twell_pack(a_s, tile_n, C)
    dense, ell, dns = O.route(c, C)
    assert 0 < dns.size < T, "fixture must route some rows each way"
    y_h = O.hybrid_forward(x, wg, wu, wd, c, i, v, tile_n, C)
    cf, i_f, vf = O.twell_pack(a_s, tile_n, tile_n)
    y_full = O.twell_forward(x, cf, i_f, vf, tile_n, wu, wd)
    # dense rows: equal to the ELL path with nothing dropped, up to float64 summation order
    np.testing.assert_allclose(y_h[dns], y_full[dns], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(y_h[ell], O.twell_forward(x[ell], c[ell], i[ell], v[ell], tile_n, wu, wd))


# ----------------------------------------------------------------------------- backward
def _fd_case(seed):
    """Tiny case with ~30% density and no pre-activation or active h near a kink."""
    for s in range(seed * 1000, seed * 1000 + 1000):
        rng = np.random.default_rng(s)
        T, d, F = 8, 16, 32
        x = rng.standard_normal((T, d))
        x[:, 0] = 1.0
        wg = rng.standard_normal((F, d)) / 4
        wg[:, 0] = -0.5
        wu = rng.standard_normal((F, d)) / 4
        wd = rng.standard_normal((F, d)) / 4
        dy = rng.standard_normal((T, d))
        f = O.ffn_forward(x, wg, wu, wd)
        act = f["g"] > 0
        if np.abs(f["g"]).min() > 1e-3 and (not act.any() or np.abs(f["h"][act]).min() > 1e-3) \
                and 0.1 < act.mean() < 0.6:
            return x, wg, wu, wd, dy
    raise RuntimeError("no kink-free case found")


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("l1", [0.0, 2e-5, 0.3])
def test_backward_finite_differences(seed, l1):
    x, wg, wu, wd, dy = _fd_case(seed)
    grads = O.ffn_backward(x, wg, wu, wd, dy, l1)
    eps = 1e-6
    params = {"dx": x, "dw_gate_t": wg, "dw_up_t": wu, "dw_down": wd}
    for name, P in params.items():
        fd = np.zeros_like(P)
        for ix in np.ndindex(P.shape):
            old = P[ix]
            P[ix] = old + eps
            lp = O.ffn_loss(x, wg, wu, wd, dy, l1)
            P[ix] = old - eps
            lm = O.ffn_loss(x, wg, wu, wd, dy, l1)
            P[ix] = old
            fd[ix] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grads[name])) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_zero_dy_closed_form():
    x, wg, wu, wd, _ = _fd_case(3)
    l1 = 0.01
    g = O.ffn_backward(x, wg, wu, wd, np.zeros_like(x), l1)
    assert np.all(g["dw_down"] == 0.0)
    np.testing.assert_array_equal(g["dh"], l1 * np.sign(g["h"]))


def test_backward_identity_closed_form():
    rng = np.random.default_rng(19)
    n = 32
    x = rng.standard_normal((7, n))
    dy = rng.standard_normal((7, n))
    I = np.eye(n)
    l1 = 0.05
    g = O.ffn_backward(x, I, I, I, dy, l1)
    np.testing.assert_allclose(g["dx"], np.where(x > 0, 2 * x * (dy + l1), 0.0), rtol=1e-14, atol=1e-15)


def test_backward_active_mask_override_matches_default():
    x, wg, wu, wd, dy = _fd_case(4)
    g0 = O.ffn_backward(x, wg, wu, wd, dy, 2e-5)
    g1 = O.ffn_backward(x, wg, wu, wd, dy, 2e-5, active=(x @ wg.T) > 0)
    for k in ("dx", "dw_gate_t", "dw_up_t", "dw_down"):
        np.testing.assert_array_equal(g0[k], g1[k])


# ----------------------------------------------------------------------------- error model
def _gate_case(T=96, d=2048, F=1024, seed=3):
    """Inputs shaped and distributed like the 2B-class bench workload (bf16,
    column-0 density offset), drawn by the shared generator."""
    from activation_sparse_feedforward_amd import workloads as W
    inp = W.make_inputs(W.workload(3, T=T, d_model=d, d_ff=F, rho=0.02))
    return inp["x"].astype(np.float32), inp["w_gate_t"].astype(np.float32)


def _f32_gate(x, w, order, truncate=False):
    """A float32 gate the way a kernel could compute it: products exact
    (bf16 x bf16 fits float32), running sums rounded to float32 after every
    term, in the given K order; ``truncate`` rounds toward zero instead of to
    nearest.  Returns ReLU(g) rounded to bf16 (float64 values)."""
    acc = np.zeros((x.shape[0], w.shape[0]), np.float32)
    for k in order:
        exact = acc.astype(np.float64) + x[:, k:k + 1].astype(np.float64) * w[None, :, k].astype(np.float64)
        r = exact.astype(np.float32)
        if truncate:
            over = np.abs(r.astype(np.float64)) > np.abs(exact)
            r = np.where(over, np.nextafter(r, np.float32(0)), r)
        acc = r
    return O.round_to_storage(np.where(acc > 0, acc, 0).astype(np.float64), "bf16")


def test_gate_error_bound_holds_for_float32_accumulation():
    """The bound covers a float32 accumulation in any order, rounded to nearest
    or truncated, followed by bf16 rounding of ReLU(g)."""
    x, w = _gate_case(T=32, d=1024, F=256)
    a_ref = O.ffn_forward(x, w, w, np.zeros(w.shape))["a"]
    bound = O.gate_error_bound(x, w, "bf16")
    d = x.shape[1]
    perm = np.random.default_rng(5).permutation(d)
    for order, trunc in ((reversed(range(d)), False), (perm, False), (range(d), True), (perm, True)):
        a_k = _f32_gate(x, w, list(order), truncate=trunc)
        assert np.all(np.abs(a_k - a_ref) <= bound)


def _outside_frac(a_wrong, a_ref, bound):
    live = (a_ref != 0) | (a_wrong != 0)
    assert live.sum() > 200
    return float(np.mean(np.abs(a_wrong - a_ref)[live] > bound[live]))


@pytest.mark.parametrize("k_slice", [1, 13, 31])
def test_gate_error_bound_rejects_a_dropped_k_slice(k_slice):
    """A gate GEMM that skips one 64-wide K slice (the main loop's step) must
    fall outside the bound on at least 90% of the active entries."""
    x, w = _gate_case()
    a_ref = O.ffn_forward(x, w, w, np.zeros(w.shape))["a"]
    keep = np.ones(x.shape[1], bool)
    keep[64 * k_slice:64 * (k_slice + 1)] = False
    a_wrong = O.round_to_storage(np.maximum((x[:, keep].astype(np.float64) @ w[:, keep].T.astype(np.float64)), 0),
                                 "bf16")
    assert _outside_frac(a_wrong, a_ref, O.gate_error_bound(x, w, "bf16")) >= 0.90


def test_gate_error_bound_rejects_transposed_weights():
    """A gate GEMM that reads W_gate^T transposed (square d_model = d_ff) must
    fall outside the bound on at least 90% of the active entries."""
    x, w = _gate_case(d=1024, F=1024)
    a_ref = O.ffn_forward(x, w, w, np.zeros(w.shape))["a"]
    a_wrong = O.round_to_storage(np.maximum(x.astype(np.float64) @ w.astype(np.float64), 0), "bf16")
    assert _outside_frac(a_wrong, a_ref, O.gate_error_bound(x, w, "bf16")) >= 0.90


def test_gate_error_bound_storage_term_scales_with_the_value():
    """The storage term is half a bf16 ulp of the value itself (2^-8 |g|), not of
    the sum of absolute products: for one exact product the bound reduces to it."""
    x = np.array([[1.5]], np.float32)
    w = np.array([[0.75], [-0.75]], np.float32)
    b = O.gate_error_bound(x, w, "bf16")
    acc = 1 * 2.0 ** -23 * 1.125 * 1.01
    np.testing.assert_allclose(b[0], acc + 2.0 ** -8 * (1.125 + acc), rtol=1e-12)
