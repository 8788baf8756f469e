"""CPU oracle for the TwELL activation-sparse gated feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library in
``activation_sparse_feedforward_amd`` never imports it, and this module imports
nothing from the library: the two share no code.  The only shared module is
the seeded input generator (``activation_sparse_feedforward_amd.workloads``),
which holds none of the arithmetic below.

Sources (the only technical page; shorthand "P2" below):
  P2 = "Sakana AI and NVIDIA introduce TwELL with CUDA kernels for 20.5%
       inference and 21.9% training" (noticias.mechatronicstore.cl), sections
       * "¿Cuál es el problema que TwELL resuelve?"      -> P2 §Problema
       * "¿Qué hace distinto a TwELL frente a ELL clásico?" -> P2 §TwELL-vs-ELL
       * "Receta de entrenamiento: dos cambios y nada más" -> P2 §Receta

What the method computes, restated:
  * the FFN is gated, with ReLU as the gate activation (P2 §Receta):
        y = (ReLU(x W_gate) * (x W_up)) W_down
  * training adds an L1 penalty on the hidden activations (P2 §Receta);
  * TwELL stores the ReLU output tile by tile: the columns are cut into tiles
    of width T_n and each (row, tile) keeps its non-zeros packed locally
    (P2 §TwELL-vs-ELL);
  * the fused inference kernel consumes TwELL and does up and down together;
    the hybrid training format sends rows with too many non-zeros to a dense
    fallback (P2 §TwELL-vs-ELL).
The method reaches the dense result exactly (only faster), so this oracle *is*
the plain dense gated FFN, plus a packer/unpacker, a router and a manual
backward.

Conventions (readings where the pages are silent):
  * Weights are stored one row per neuron: W_gate^T, W_up^T, W_down are each
    [d_ff x d_model] row-major, so g = x @ W_gate^T.T, y = h @ W_down.
  * Arithmetic is float64 throughout; the pages fix no precision.  Inputs are
    float32 arrays holding exact bf16 / fp32 values.
  * ReLU'(0) = 0 and sign(0) = 0; g <= 0 is inactive.
  * TwELL of an activation matrix A (values already rounded to the storage
    dtype): per (row t, tile b) count = #non-zeros, slots s < min(count, C)
    hold the non-zeros in ascending column order as (tile-local index, value);
    other slots hold (0, +0.0).  count keeps the true count even when it
    exceeds C (the overflowing entries are dropped from the slots).
  * L1 acts on h = ReLU(g) * u, summed over all (t, j): loss term l1 * sum|h|.

Every function here is pinned by tests in ``tests/test_oracle.py`` against
closed forms, invariants, brute force on tiny inputs, a hand-worked golden
fixture and central finite differences.  Parity of the L1 placement and
normalisation is unpinned by the pages (they give only the coefficient); the
finite differences pin only the loss stated above.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gate_forward", "ffn_forward", "round_to_storage", "twell_pack", "twell_unpack", "twell_forward",
    "route", "hybrid_forward", "ffn_backward", "ffn_loss", "gate_error_bound",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Dense forward  [P2 §Receta: ReLU gate in a gated FFN]
# ---------------------------------------------------------------------------
def gate_forward(x, w_gate_t):
    """The gate in float64: g = x W_gate (pre-activation) and a = ReLU(g).
    The first step of ``ffn_forward`` (and of the sparse path, whose TwELL is
    the packing of a)."""
    g = _f64(x) @ _f64(w_gate_t).T
    return g, np.where(g > 0.0, g, 0.0)


def ffn_forward(x, w_gate_t, w_up_t, w_down) -> dict:
    """Plain dense gated FFN in float64.

    g = x W_gate (pre-activation), a = ReLU(g), u = x W_up, h = a * u, y = h W_down.
    Returns all intermediates as float64 arrays.
    """
    x = _f64(x)
    g, a = gate_forward(x, w_gate_t)
    u = x @ _f64(w_up_t).T
    h = a * u
    y = h @ _f64(w_down)
    return {"g": g, "a": a, "u": u, "h": h, "y": y}


def _round_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value, ties to even, in one rounding step.

    bf16 keeps 8 significant bits: a value m * 2**e (0.5 <= |m| < 1) is rounded
    to a multiple of 2**(e - 8).  Below the smallest normal (2**-126) the step
    stays at the subnormal quantum 2**-133.  Overflow past the bf16 range is
    outside every workload and is not handled.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                      # v = m * 2**e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


def round_to_storage(a, dtype: str) -> np.ndarray:
    """Round values to the TwELL storage dtype ("fp32" or "bf16"); returns float64."""
    a = _f64(a)
    if dtype == "fp32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(a)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# TwELL packing / unpacking  [P2 §TwELL-vs-ELL: tile-local packing, width T_n]
# ---------------------------------------------------------------------------
def twell_pack(a_s, tile_n: int, slots: int):
    """Pack an activation matrix A [T x F] (storage-rounded values) into TwELL.

    Returns (count int32 [T, n_t], idx uint8 [T, n_t, C], val float64 [T, n_t, C])
    with n_t = F / tile_n and C = slots.

    For every (t, b): the non-zeros of A[t, b*T_n:(b+1)*T_n] are listed in
    ascending column order; count is their number; the first min(count, C) of
    them go to slots 0.. as (column - b*T_n, value); remaining slots are (0, 0).
    """
    A = _f64(a_s)
    T, F = A.shape
    if F % tile_n:
        raise ValueError("d_ff must be a multiple of tile_n")
    n_t = F // tile_n
    tiles = A.reshape(T, n_t, tile_n)
    nz = tiles != 0.0
    count = nz.sum(axis=2).astype(np.int32)
    # rank of each non-zero inside its tile, in ascending column order
    rank = np.cumsum(nz, axis=2) - 1
    keep = nz & (rank < slots)
    t_i, b_i, c_i = np.nonzero(keep)
    s_i = rank[t_i, b_i, c_i]
    idx = np.zeros((T, n_t, slots), dtype=np.uint8)
    val = np.zeros((T, n_t, slots), dtype=np.float64)
    idx[t_i, b_i, s_i] = c_i.astype(np.uint8)
    val[t_i, b_i, s_i] = tiles[t_i, b_i, c_i]
    return count, idx, val


def twell_unpack(count, idx, val, tile_n: int) -> np.ndarray:
    """Scatter TwELL back to a dense [T x F] matrix (float64).

    Only the slots s < min(count, C) are scattered; the rest of the row is zero.
    When no tile overflows this is the exact inverse of ``twell_pack``.
    """
    count = np.asarray(count)
    idx = np.asarray(idx)
    val = _f64(val)
    T, n_t, C = idx.shape
    A = np.zeros((T, n_t, tile_n), dtype=np.float64)
    live = np.arange(C)[None, None, :] < np.minimum(count, C)[:, :, None]
    t_i, b_i, s_i = np.nonzero(live)
    A[t_i, b_i, idx[t_i, b_i, s_i].astype(np.int64)] = val[t_i, b_i, s_i]
    return A.reshape(T, n_t * tile_n)


def twell_forward(x, count, idx, val, tile_n: int, w_up_t, w_down) -> np.ndarray:
    """Fused up+down on TwELL input  [P2 §TwELL-vs-ELL: inference kernel].

    For each row t and each stored slot (neuron j, value a):
        u = x[t] . W_up^T[j],  h = a * u,  y[t] += h * W_down[j]
    written as its dense equivalent: y = (unpack(TwELL) * (x W_up)) W_down.
    Overflowing tiles contribute only their stored slots.
    """
    a_twell = twell_unpack(count, idx, val, tile_n)
    u = _f64(x) @ _f64(w_up_t).T
    return (a_twell * u) @ _f64(w_down)


# ---------------------------------------------------------------------------
# Hybrid routing  [P2 §TwELL-vs-ELL: rows with too many non-zeros go dense]
# ---------------------------------------------------------------------------
def route(count, slots: int):
    """Row router: a row is dense iff any of its tiles has count > C.

    Returns (dense bool [T], ell_rows int32 ascending, dense_rows int32 ascending).
    """
    count = np.asarray(count)
    dense = (count > slots).any(axis=1) if count.size else np.zeros(count.shape[0], bool)
    ell_rows = np.nonzero(~dense)[0].astype(np.int32)
    dense_rows = np.nonzero(dense)[0].astype(np.int32)
    return dense, ell_rows, dense_rows


def hybrid_forward(x, w_gate_t, w_up_t, w_down, count, idx, val, tile_n: int, slots: int) -> np.ndarray:
    """Hybrid forward: ELL rows through the TwELL path, dense rows through the dense FFN."""
    dense, ell_rows, dense_rows = route(count, slots)
    x = _f64(x)
    y = np.zeros((x.shape[0], _f64(w_down).shape[1]), dtype=np.float64)
    if ell_rows.size:
        y[ell_rows] = twell_forward(x[ell_rows], count[ell_rows], idx[ell_rows], val[ell_rows],
                                    tile_n, w_up_t, w_down)
    if dense_rows.size:
        y[dense_rows] = ffn_forward(x[dense_rows], w_gate_t, w_up_t, w_down)["y"]
    return y


# ---------------------------------------------------------------------------
# Backward with the L1 activation penalty  [P2 §Receta]
# ---------------------------------------------------------------------------
def ffn_loss(x, w_gate_t, w_up_t, w_down, dy, l1_coef: float) -> float:
    """Scalar L = sum(y * dy) + l1 * sum|h|, whose gradients ``ffn_backward`` returns."""
    f = ffn_forward(x, w_gate_t, w_up_t, w_down)
    return float(np.sum(f["y"] * _f64(dy)) + l1_coef * np.sum(np.abs(f["h"])))


def ffn_backward(x, w_gate_t, w_up_t, w_down, dy, l1_coef: float, active=None) -> dict:
    """Manual backward of ``ffn_loss`` in float64.

    dh = dy W_down^T + l1 * sign(h)          (sign(0) = 0)
    du = dh * a ;  dg = dh * u * [g > 0]
    dx[t,k] = sum_j dg[t,j] W_gate^T[j,k] + du[t,j] W_up^T[j,k]
    dW_gate^T = dg^T x ;  dW_up^T = du^T x ;  dW_down = h^T dy

    ``active`` (bool [T x F], optional) replaces the decision g > 0.  It lets a
    parity test take the activation mask from the kernel under test, so that a
    pre-activation within rounding of zero is decided the same way on both
    sides; the values stay this oracle's float64 ones.
    """
    x = _f64(x)
    wg, wu, wd, dy = _f64(w_gate_t), _f64(w_up_t), _f64(w_down), _f64(dy)
    g = x @ wg.T
    on = (g > 0.0) if active is None else np.asarray(active, dtype=bool)
    a = np.where(on, g, 0.0)
    u = x @ wu.T
    h = a * u
    dh = dy @ wd.T + l1_coef * np.sign(h)
    du = dh * a
    dg = np.where(on, dh * u, 0.0)
    dx = dg @ wg + du @ wu
    return {
        "dx": dx,
        "dw_gate_t": dg.T @ x,
        "dw_up_t": du.T @ x,
        "dw_down": h.T @ dy,
        "dh": dh, "dg": dg, "du": du, "h": h, "a": a, "u": u, "g": g,
    }


# ---------------------------------------------------------------------------
# Error model used by parity tests
# ---------------------------------------------------------------------------
def gate_error_bound(x, w_gate_t, dtype: str, rows=None) -> np.ndarray:
    """Elementwise bound on |a_kernel - ReLU(g)| for a kernel that accumulates
    g in float32 over d_model terms (any order) and stores ReLU(g) in ``dtype``.

    Accumulation: with S = sum_k |x_k w_k|, each of the K roundings of a
    float32 dot product (the products, then the running sums) moves the result
    by at most one float32 ulp, i.e. 2^-23 relative, which covers a matrix
    unit that rounds to nearest as well as one that truncates; to first order
        |g_kernel - g| <= acc = K * 2^-23 * S   (times 1.01 for the higher terms).
    Storage: rounding g_kernel to bf16 (nearest, ties to even) moves it by at
    most half a bf16 ulp, 2^-8 |g_kernel| <= 2^-8 (|g| + acc); float32 storage
    keeps the accumulator (2^-24 is used).  ReLU is 1-Lipschitz, so
        |a_kernel - ReLU(g)| <= acc + rel * (|g| + acc).
    """
    x = _f64(x) if rows is None else _f64(x)[rows]
    w = _f64(w_gate_t)
    K = x.shape[1]
    s = np.abs(x) @ np.abs(w).T
    g = np.abs(x @ w.T)
    acc = (K * 2.0 ** -23) * s * 1.01
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    return acc + rel * (g + acc) + 1e-30
