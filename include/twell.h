/*
 * twell.h -- C ABI of libtwell: the TwELL activation-sparse gated FFN on MI355X (gfx950).
 *
 * The layer is  y = (ReLU(x W_gate) * (x W_up)) W_down  with a ReLU gate, whose
 * output is mostly exact zeros.  Sources: the page "Sakana AI and NVIDIA
 * introduce TwELL with CUDA kernels for 20.5% inference and 21.9% training"
 * (noticias.mechatronicstore.cl), called P2 below, sections
 *   "¿Qué hace distinto a TwELL frente a ELL clásico?"  (P2 §TwELL-vs-ELL):
 *       tile-local packing built in the gate matmul's epilogue, the fused
 *       up/down inference kernel, the hybrid ELL / dense-fallback format;
 *   "Receta de entrenamiento: dos cambios y nada más"  (P2 §Receta):
 *       ReLU gate, L1 penalty on the hidden activations;
 *   "¿Cuál es el problema que TwELL resuelve?"  (P2 §Problema):
 *       the dense Tensor-Core FFN that the sparse path is measured against.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layouts (all row-major, contiguous):
 *      x, y, dy, dx     [T x d_model]          dtype
 *      w_gate_t         [d_ff x d_model]        dtype   row j = neuron j's gate weights
 *      w_up_t           [d_ff x d_model]        dtype   row j = neuron j's up weights
 *      w_down           [d_ff x d_model]        dtype   row j = neuron j's output row
 *    so g = x . w_gate_t^T, u = x . w_up_t^T, y = h . w_down.
 *  - TwELL (twell_act), with n_t = d_ff / tile_n and C = slots:
 *      count  int32  [T][n_t]        number of non-zeros of ReLU(g) in the (row, tile),
 *                                    the TRUE number even when it exceeds C;
 *      idx    uint8  [T][n_t][C]     tile-local column (0..tile_n-1) of each stored non-zero;
 *      val    dtype  [T][n_t][C]     its value ReLU(g) rounded to dtype.
 *    Slots s < min(count, C) hold the non-zeros in ascending column order; the
 *    others hold idx 0 and value +0.  A value is a non-zero iff its rounded
 *    (stored) value is not zero.
 *  - Pointers: every array argument is a DEVICE pointer, 16-byte aligned,
 *    owned by the caller.  The library never allocates or frees memory;
 *    scratch memory is passed in as `ws`, except by the allocation-free
 *    twell_ffn_fwd_hybrid_noalloc, whose scratch is a static device array.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = default
 *    stream).  All calls are asynchronous: they return after host-side
 *    validation and the kernel launches, with no host synchronisation.
 *  - Errors: TWELL_EINVAL for a bad descriptor, NULL / misaligned pointer or
 *    too-small workspace (nothing is launched); TWELL_EUNSUPPORTED for a valid
 *    shape the library has no kernel for; TWELL_EHIP when a launch fails;
 *    TWELL_ESCRATCH when a problem exceeds the allocation-free entry point's
 *    static scratch (nothing is launched).
 *    Data-dependent conditions (overflowing tiles, dense-row cap exceeded) are
 *    reported in device counters, never as host errors.
 *  - Supported shapes: dtype BF16 with d_model % 512 == 0 and d_model <= 4096,
 *    or FP32 with d_model % 256 == 0 and d_model <= 2048; tile_n in {64, 128};
 *    d_ff % tile_n == 0; 1 <= slots <= tile_n; T >= 0 (T == 0 is a no-op);
 *    T * max(d_model, d_ff) < 2^31.
 *  - Threading: calls are thread-safe (the shared state is a per-device cache
 *    of the CU count and of the scratch address, held in atomics), except that
 *    calls of twell_ffn_fwd_hybrid_noalloc must not overlap on one device.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TWELL_OK = 0,
  TWELL_EINVAL = 1,
  TWELL_EUNSUPPORTED = 2,
  TWELL_EHIP = 3,
  TWELL_ESCRATCH = 4 /* the problem needs more scratch than the allocation-free entry point holds */
} twell_status;

typedef enum { TWELL_FP32 = 0, TWELL_BF16 = 1 } twell_dtype;

/* Problem descriptor.  T = tokens, d_model / d_ff = FFN widths, tile_n = TwELL
 * tile width T_n (the gate matmul's N tile), slots = C. */
typedef struct {
  int64_t T;
  int32_t d_model;
  int32_t d_ff;
  int32_t tile_n;
  int32_t slots;
  int32_t dtype; /* twell_dtype */
} twell_desc;

/* The three TwELL planes (device pointers, layouts above). */
typedef struct {
  int32_t* count;
  uint8_t* idx;
  void* val;
} twell_act;

/* Row routing of the hybrid format (device arrays owned by the caller).
 * Written by twell_ffn_fwd_hybrid; read by the backward. */
typedef struct {
  int32_t* ell_rows;      /* [T]               rows served from TwELL, ascending           */
  int32_t* dense_rows;    /* [max_dense_rows]  rows served by the dense fallback, ascending */
  int32_t* n_rows;        /* [3]  {n_ell, n_dense, dense rows beyond max_dense_rows}        */
  uint8_t* row_kind;      /* [T]  1 = row went to the dense fallback, 0 = TwELL             */
  int64_t max_dense_rows; /* capacity of dense_rows and of the fallback workspace           */
} twell_route;

/* Byte sizes of the TwELL planes and of the workspaces, for a descriptor. */
typedef struct {
  size_t count;        /* T * n_t * 4                                        */
  size_t idx;          /* T * n_t * C                                        */
  size_t val;          /* T * n_t * C * sizeof(dtype)                        */
  size_t ws_dense_fwd; /* twell_dense_ffn_fwd: h [T x d_ff] + W_down^T         */
  size_t ws_hybrid;    /* workspace of twell_ffn_fwd_hybrid (max_dense_rows)  */
  size_t ws_bwd;       /* workspace of twell_ffn_bwd (max_dense_rows)         */
  size_t ws_pack_classic; /* twell_pack_classic: dense ReLU(g) [T x d_ff]      */
} twell_sizes_t;

/* Fill *out for descriptor *d and a dense-row capacity (>= 0).  Host only.
 * Returns TWELL_EINVAL / TWELL_EUNSUPPORTED like the compute calls would. */
twell_status twell_sizes(const twell_desc* d, int64_t max_dense_rows, twell_sizes_t* out);

/* Gate GEMM + ReLU + TwELL pack, in ONE kernel dispatch.
 * [P2 §TwELL-vs-ELL: the sparse format is produced inside the epilogue of the
 * gate matmul, with no extra launch and no dense write of the activations.]
 *   x [T x d_model], w_gate_t [d_ff x d_model] (dtype)  ->  act (all three planes written).
 * g accumulates in fp32; ReLU(g) is rounded to dtype before the non-zero test.
 * stats  (device int64[2], nullable): ACCUMULATED (atomic add) with
 *        [0] += number of (row, tile) pairs whose count exceeds slots,
 *        [1] += sum of all counts (= non-zeros of ReLU(g));  zero it first.
 * gate_dbg (device, nullable): if given, the same kernel also writes the dense
 *        ReLU(g) [T x d_ff] in dtype (parity / debugging only; it is the dense
 *        write-back the method exists to avoid, so leave it NULL when timing). */
twell_status twell_pack(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                        int64_t* stats, void* gate_dbg, void* stream);

/* The same TwELL planes built the classic way, as a baseline for twell_pack:
 * [P2 §Problema and §TwELL-vs-ELL: converting a dense activation tensor to a
 * sparse format in a separate kernel costs an extra launch and a full write
 * and read of that tensor, which eats the saving.]
 * Kernel 1: the gate GEMM (same accumulation order as twell_pack) writes
 *           ReLU(g) rounded to dtype densely into ws, [T x d_ff];
 * Kernel 2: one wave per (row, tile) converts it to TwELL.
 * act is written exactly as twell_pack writes it (byte-identical planes).
 * ws: twell_sizes().ws_pack_classic bytes. */
twell_status twell_pack_classic(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                                void* ws, size_t ws_bytes, void* stream);

/* Fused up + down projection on TwELL input: one fused kernel, the
 * intermediate never written to memory.
 * [P2 §TwELL-vs-ELL: one fused kernel reads TwELL and runs the up and down
 * projections together; the intermediate never reaches global memory.]
 * Dispatches, by batch size T and row width d_model: below 2048 rows a
 * one-workgroup-per-row kernel (16 waves; 8 for bf16 rows wider than 2048), in
 * ONE dispatch; a one-wave-per-row kernel, in ONE dispatch, for fp32 rows
 * wider than 1024 and for bf16 rows wider than 2048 from 2048 to 4095 rows.
 * All other batches take the lockstep kernel (workgroups of W waves --
 * 16, or 8 for bf16 rows wider than 2048 -- that sweep the neuron tiles
 * together, each wave holding R rows: as many as its registers, the
 * workgroup's LDS and the per-wave list allow -- 2 at d_model = 2048 and at
 * 2560 .. 4096, 4 at d_model <= 1024 when C <= 32 -- but fewer while that
 * would leave CUs without a workgroup), dispatched once per generation of
 * workgroups the device runs at once (one per CU), on disjoint row blocks:
 * ceil(ceil(T / (W R)) / CUs) dispatches of the same kernel, e.g. 2 at
 * T = 16384, d_model = 2048 (W = 16, R = 2), 1 at T = 8192, d_model = 1024
 * (R = 2) and 4 at T = 16384, d_model = 4096 (W = 8, R = 2) on a 256-CU
 * MI355X.  Every row is computed start to finish by one workgroup of one
 * dispatch; a workgroup deals its rows to its waves by their entry counts (a
 * row's result does not depend on the wave).
 * Bits: each row's tiles are summed starting at a chunk that depends on its
 * workgroup's index and generation, hence on the device's CU count; y is
 * bitwise reproducible on one device (and on devices with the same CU count),
 * and within the stated tolerance elsewhere.
 * For every row t and stored slot (neuron j = b*tile_n + idx, value a):
 *   u = x[t] . w_up_t[j];  h = a * u;  y[t] += h * w_down[j]   (fp32 accumulate)
 * y [T x d_model] is overwritten (stored in dtype).  A tile with count > slots
 * contributes only its stored slots (the plain format is lossy there; the
 * hybrid entry point is the remedy). */
twell_status twell_ffn_fwd(const twell_desc* d, const void* x, twell_act act, const void* w_up_t,
                           const void* w_down, void* y, void* stream);

/* Hybrid forward: row router + fused TwELL path on ELL rows + dense MFMA
 * fallback on dense rows.  [P2 §TwELL-vs-ELL: for training, whose sparsity is
 * far from uniform, each row goes at run time either to a compact ELL store
 * or to a dense fallback when it has too many non-zeros.]
 * act must come from twell_pack on the same x and w_gate_t.
 * Kernels (same stream, no host synchronisation):
 *   1-2. router: a row is dense iff some tile has count > slots; ascending
 *        ell_rows / dense_rows, n_rows, row_kind.  At most max_dense_rows
 *        rows are kept dense; further dense rows are served (lossily) from
 *        TwELL and counted in n_rows[2].
 *   3.   fused up/down (as twell_ffn_fwd) over ell_rows; ELL rows with far
 *        more non-zeros than the batch's mean row (> max(2 slots, 2 x mean),
 *        at most 1024 of them) are cut into tile ranges processed in parallel
 *        and summed in a fixed order; the other ELL rows are dealt over
 *        windows of 8 lockstep workgroups by their entry counts.  Which
 *        workgroup computes a row therefore differs from twell_ffn_fwd, so its
 *        y can differ in the last bits (deterministic either way);
 *   4-5. dense gate|up GEMM over the gathered dense rows (h = ReLU(g) * u,
 *        recomputed, kept in ws), then the down GEMM scattered into y.
 * y [T x d_model] is overwritten.  ws: twell_sizes(d, max_dense_rows).ws_hybrid bytes. */
twell_status twell_ffn_fwd_hybrid(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                                  const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                                  void* ws, size_t ws_bytes, void* stream);

/* Backward of the hybrid-format FFN, reusing the forward's TwELL and route.
 * [P2 §Receta: ReLU gate and an L1 term on the hidden activations;
 *  P2 §TwELL-vs-ELL: the training format is the hybrid one.]
 * Loss whose gradients are returned:  L = sum(y * dy) + l1_coef * sum|h|,
 * with h = ReLU(g) * u the hidden activation feeding w_down (sign(0) = 0,
 * ReLU'(0) = 0).  Given dy [T x d_model] (dtype):
 *   dx        [T x d_model]  dtype, overwritten (every row);
 *   dw_gate_t, dw_up_t, dw_down  [d_ff x d_model] fp32, overwritten.
 * act and route must be those of the twell_pack / twell_ffn_fwd_hybrid call on
 * the same x.  Rows in route->ell_rows use only their stored TwELL slots (a
 * row the forward served lossily from TwELL is differentiated the same way);
 * rows in route->dense_rows are recomputed densely on MFMA.
 * Deterministic: each neuron's weight gradient is the sum of its ELL rows'
 * terms in ascending token order, plus the dense rows' GEMM result (bitwise
 * the same on any device).  dx of the ELL rows comes from
 * a lockstep kernel dispatched once per generation of resident workgroups like
 * twell_ffn_fwd's (16 waves per workgroup, 8 for bf16 rows wider than 2048,
 * which take it from 4096 rows on and one wave per row below; fp32 rows wider
 * than 1024 always one wave per row), with the same dependence of its bits on
 * the CU count.
 * ws: twell_sizes(d, route->max_dense_rows).ws_bwd bytes. */
twell_status twell_ffn_bwd(const twell_desc* d, const void* x, twell_act act, const twell_route* route,
                           const void* w_gate_t, const void* w_up_t, const void* w_down, const void* dy,
                           float l1_coef, void* dx, float* dw_gate_t, float* dw_up_t, float* dw_down,
                           void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch array of twell_ffn_fwd_hybrid_noalloc
 * (one copy per device the library runs on, held until the process ends). */
#define TWELL_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* twell_ffn_fwd_hybrid without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels, results (bit for
 * bit) and route outputs as twell_ffn_fwd_hybrid; its workspace is instead a
 * static device array of TWELL_NOALLOC_SCRATCH_BYTES per device, whose device
 * address is looked up (hipGetSymbolAddress) on the first call on each
 * device.  It calls no hipMalloc / hipFree and allocates nothing.
 *   Limit: twell_sizes(d, route->max_dense_rows).ws_hybrid must not exceed
 *   TWELL_NOALLOC_SCRATCH_BYTES, else TWELL_ESCRATCH is returned and nothing
 *   is launched (e.g. the 2B-class shape, T = 16384, d_model = 2048,
 *   d_ff = 8192, fits with max_dense_rows up to 454).
 *   Every call on a device shares that device's array: calls that overlap on
 *   one device (other streams, other threads) race and must not be issued.
 *   The array keeps the last call's contents; no part of it needs to start
 *   at zero (every workspace entry is written before it is read). */
twell_status twell_ffn_fwd_hybrid_noalloc(const twell_desc* d, const void* x, const void* w_gate_t,
                                          twell_act act, const void* w_up_t, const void* w_down, void* y,
                                          const twell_route* route, void* stream);

/* The library's own dense MFMA FFN, the baseline the sparse path is compared with.
 * [P2 §Problema: GPUs are built for dense matrix products; the sparse path must
 * beat the dense one.]
 * Kernel 1: W_down^T [d_model x d_ff] written into ws (after h, 256-byte aligned);
 * Kernel 2: g = x w_gate, u = x w_up in one GEMM, epilogue h = ReLU(g) * u
 *           stored to ws as dtype [T x d_ff];
 * Kernel 3: y = h w_down (y overwritten, dtype).
 * ws must hold twell_sizes().ws_dense_fwd bytes. */
twell_status twell_dense_ffn_fwd(const twell_desc* d, const void* x, const void* w_gate_t,
                                 const void* w_up_t, const void* w_down, void* y, void* ws,
                                 size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* twell_status_str(twell_status s);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
