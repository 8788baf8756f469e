"""Seeded synthetic workloads for the TwELL gated FFN.

This module only draws and rounds inputs; it holds none of the FFN's arithmetic.
Both the HIP path (through bench.py and the GPU tests) and the CPU oracle consume
the arrays it returns, so the two sides always see bit-identical inputs.

Recipe (stated once here, repeated in the design notes):

* Every array is drawn with NumPy's PCG64, ``default_rng([config_id, stream])``,
  one stream per tensor: x=1, W_gate^T=2, W_up^T=3, W_down=4, dy=5, per-row
  density=6.  Draws are float32; bf16 workloads then round each value once to
  bf16 (round-to-nearest-even) and the rounded values ARE the inputs.
* x ~ N(0, 1); W_gate^T, W_up^T ~ N(0, 1/d_model) stored [d_ff x d_model];
  W_down ~ N(0, 1/d_ff) stored [d_ff x d_model].  Row j of each is neuron j.
* Gate density is set with one input feature (column 0): x[t, 0] = c_t and
  W_gate^T[j, 0] = -||W_gate^T[j, 1:]||, so g[t, j] ~ N(-c_t s_j, s_j^2) and
  P(g > 0) = 1 - Phi(c_t) = rho_t exactly for every neuron (before rounding).
  The tiny fp32 workload instead uses the fixed offset -2.58*sqrt(255/256) on
  W_gate^T[:, 0] with x[:, 0] = 1, giving P(g > 0) = Phi(-2.58) ~ 0.49%.
* The training workload draws rho_t per row: with probability 0.98 a lognormal
  0.005*exp(0.5 Z), otherwise (a 2% tail) U(5%, 20%).

These synthetic activations stand in for the pages' L1-trained 2B-model
activations, which need trained weights that do not exist here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
from scipy.special import ndtri

STREAM_X, STREAM_WG, STREAM_WU, STREAM_WD, STREAM_DY, STREAM_RHO = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic FFN problem: shapes, dtype, TwELL tile geometry, density."""

    config_id: int
    name: str
    T: int
    d_model: int
    d_ff: int
    dtype: str          # "fp32" or "bf16"
    tile_n: int
    slots: int
    density: str        # "offset258" | "uniform" | "lognormal_tail"
    rho: float = 0.005  # target gate density for "uniform"
    l1_coef: float = 2e-5


# The five workloads.  C = 16 slots per 128-wide tile is stated for the
# training workload only; it is used for the other bf16 workloads as well so
# that there is one format.
WORKLOADS = {
    1: Workload(1, "tiny_fp32_T256_d256_F1024", 256, 256, 1024, "fp32", 64, 8, "offset258"),
    2: Workload(2, "llama0.5B_ffn_T8192_d1024_F4096", 8192, 1024, 4096, "bf16", 128, 16, "uniform"),
    3: Workload(3, "llama2B_ffn_T16384_d2048_F8192", 16384, 2048, 8192, "bf16", 128, 16, "uniform"),
    4: Workload(4, "llama2B_ffn_train_T16384_d2048_F8192_lognormal", 16384, 2048, 8192, "bf16", 128, 16,
                "lognormal_tail"),
    5: Workload(5, "llama2B_ffn_sweep_T16384_d2048_F8192", 16384, 2048, 8192, "bf16", 128, 16, "uniform"),
}

SWEEP_RHOS = (0.001, 0.005, 0.01, 0.02, 0.05)


def workload(config_id: int, *, T: Optional[int] = None, rho: Optional[float] = None,
             d_model: Optional[int] = None, d_ff: Optional[int] = None) -> Workload:
    """Return a workload, optionally with T / rho / widths overridden (smaller test shapes)."""
    w = WORKLOADS[config_id]
    kw = {}
    if T is not None:
        kw["T"] = int(T)
    if rho is not None:
        kw["rho"] = float(rho)
    if d_model is not None:
        kw["d_model"] = int(d_model)
    if d_ff is not None:
        kw["d_ff"] = int(d_ff)
    return dataclasses.replace(w, **kw) if kw else w


def round_f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly equal float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.default_rng([w.config_id, stream])


def _normal(w: Workload, stream: int, shape, scale: float) -> np.ndarray:
    a = _rng(w, stream).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def row_densities(w: Workload) -> np.ndarray:
    """Per-row target gate density rho_t (float64, length T)."""
    if w.density == "uniform":
        return np.full(w.T, w.rho, dtype=np.float64)
    if w.density == "lognormal_tail":
        rng = _rng(w, STREAM_RHO)
        z = rng.standard_normal(w.T)
        tail = rng.random(w.T) < 0.02
        tail_rho = rng.uniform(0.05, 0.20, w.T)
        rho = np.where(tail, tail_rho, 0.005 * np.exp(0.5 * z))
        return np.clip(rho, 1e-6, 0.5)
    if w.density == "offset258":
        from scipy.special import ndtr
        return np.full(w.T, float(ndtr(-2.58)), dtype=np.float64)
    raise ValueError(w.density)


def _to_dtype(a: np.ndarray, dtype: str):
    """Round once to the workload dtype; return (float32 values, raw storage array)."""
    if dtype == "fp32":
        a = np.ascontiguousarray(a, dtype=np.float32)
        return a, a
    bits = round_f32_to_bf16_bits(a)
    return bf16_bits_to_f32(bits), bits


def make_inputs(w: Workload, *, with_dy: bool = False) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with, for each tensor name in (x, w_gate_t, w_up_t, w_down[, dy]):
      ``name``         float32 values (exactly representable in the workload dtype)
      ``name + '_raw'`` the storage array: float32 for fp32, uint16 bf16 bits for bf16
    plus ``rho_rows`` (the per-row target densities) and ``workload``.
    """
    T, d, F = w.T, w.d_model, w.d_ff
    x = _normal(w, STREAM_X, (T, d), 1.0)
    wg = _normal(w, STREAM_WG, (F, d), 1.0 / np.sqrt(d))
    wu = _normal(w, STREAM_WU, (F, d), 1.0 / np.sqrt(d))
    wd = _normal(w, STREAM_WD, (F, d), 1.0 / np.sqrt(F))
    rho = row_densities(w)
    if w.density == "offset258":
        x[:, 0] = 1.0
        wg[:, 0] = np.float32(-2.58 * np.sqrt(255.0 / 256.0))
    else:
        wg[:, 0] = -np.sqrt(np.sum(wg[:, 1:].astype(np.float64) ** 2, axis=1)).astype(np.float32)
        x[:, 0] = ndtri(1.0 - rho).astype(np.float32)
    out = {"workload": w, "rho_rows": rho}
    tensors = {"x": x, "w_gate_t": wg, "w_up_t": wu, "w_down": wd}
    if with_dy:
        tensors["dy"] = _normal(w, STREAM_DY, (T, d), 1.0)
    for k, v in tensors.items():
        vals, raw = _to_dtype(v, w.dtype)
        out[k] = vals
        out[k + "_raw"] = raw
    return out
