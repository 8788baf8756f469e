// Kernel argument blocks and launch functions shared between the kernel
// translation units and the C-ABI layer (host code only sees these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

struct PackArgs {
  const void* x;         // [T x d]
  const void* w_gate_t;  // [F x d]
  int64_t T;
  int32_t d, F, tile_n, C;
  int32_t* count;  // [T][n_t]
  uint8_t* idx;    // [T][n_t][C]
  void* val;       // [T][n_t][C]
  unsigned long long* stats;  // [2] or null
  void* gate_dbg;             // [T x F] or null
};

struct FusedArgs {
  const void* x;  // [T x d]
  const int32_t* count;
  const uint8_t* idx;
  const void* val;
  const void* w_up_t;  // [F x d]
  const void* w_down;  // [F x d]
  void* y;             // [T x d]
  const int32_t* rows;        // row list (ELL rows of the hybrid format) or null = all rows
  const int32_t* n_rows_dev;  // device count of `rows` or null
  const int32_t* row_total;   // [T] sum of each token's counts, or null (lockstep row balancing)
  int64_t T;                  // rows of x / y; also the upper bound of the row list
  int32_t d, F, tile_n, C;
  // split mode (launch_fused_split): every row of the list is cut into
  // `groups` tile ranges, one wave each, whose fp32 partial outputs go to
  // part[group][i_row][d] (i_row < part_rows); y is then not written.
  int32_t groups;
  float* part;
  int64_t part_rows;
  // lockstep launches (set by the launcher): workgroups the device runs at
  // once, and the first row block of this launch
  int32_t resident;
  int64_t blk0;
};

// Classic ELL construction (baseline): dense ReLU(g) [T x F] written to `dense`,
// then converted to the TwELL planes by a second kernel.
struct ClassicArgs {
  const void* x;         // [T x d]
  const void* w_gate_t;  // [F x d]
  void* dense;           // [T x F] dtype (workspace)
  int64_t T;
  int32_t d, F, tile_n, C;
  int32_t* count;
  uint8_t* idx;
  void* val;
};
// Hybrid router: flags[t] (1 = dense), ascending ell_rows / dense_rows lists,
// n_rows = {n_ell, n_dense, n_dense_over_cap}.
struct RouteArgs {
  const int32_t* count;  // [T][n_t]
  int64_t T;
  int32_t n_t, C;
  int64_t cap;           // at most this many dense rows are kept
  uint8_t* flags;        // [T] scratch; final value 1 = kept dense, 0 = ELL
  int32_t* block_dense;  // [ceil(T/256)] scratch
  int32_t* ell_rows;     // [T]
  int32_t* dense_rows;   // [cap]
  int32_t* n_rows;       // [3]
  // light / heavy split of the ELL rows (launch_route_split; null = not used)
  int32_t* row_total;    // [T] non-zeros of each row (sum of its counts)
  int32_t* block_total;  // [ceil(T/256)] sum of row_total per block
  int32_t* light_rows;   // [T]
  int32_t* heavy_rows;   // [heavy_cap]
  int32_t* split_n;      // [2] {n_light, n_heavy}
  int32_t* block_heavy;  // [ceil(T/256)] heavy rows per block of list positions
  int64_t heavy_cap;
};

// h[m, j] = ReLU(x[row(m)] . w_gate_t[j]) * (x[row(m)] . w_up_t[j]) for m < n_rows,
// where row(m) = rows ? rows[m] : m and n_rows = n_rows_dev ? *n_rows_dev : M.
struct GateUpArgs {
  const void* x;
  const void* w_gate_t;
  const void* w_up_t;
  void* h;  // [M x F] (compact rows)
  const int32_t* rows;        // gather table or null
  const int32_t* n_rows_dev;  // device row count or null
  int64_t M;                  // host row count / upper bound
  int32_t d, F;
};

// y[row(m), :] = h[m, :] . w_down  for m < n_rows (row(m) as above, scatter).
struct DownArgs {
  const void* h;         // [M x F]
  const void* w_down;    // [F x d]
  const void* w_down_t;  // [d x F] (launch_dense256: written there from w_down first)
  void* y;             // [T x d]
  const int32_t* rows;
  const int32_t* n_rows_dev;
  int64_t M;
  int32_t d, F;
  // split-K (launch_down only): splits > 1 writes fp32 partials part[split][M][d]
  // and a fixed-order reduction then rounds them into y (deterministic)
  float* part;
  int32_t splits;
};
// Split-K factor for a skinny GEMM over K (a multiple of slice elements): the
// largest s in {16, 8, 4, 2, 1} with K / s >= 512 and K / s a multiple of the
// slice, so that few M tiles still fill the chip.
inline int split_k_for(int64_t K, int slice_elems) {
  for (int s = 16; s > 1; s >>= 1)
    if (K / s >= 512 && (K / slice_elems) % s == 0) return s;
  return 1;
}

// Backward of the hybrid-format FFN (sparse rows: k_bwd.hip, dense rows: k_bwd_dense.hip).
struct BwdArgs {
  const void* x;
  const void* dy;
  const int32_t* count;
  const uint8_t* idx;
  const void* val;
  const void* w_gate_t;
  const void* w_up_t;
  const void* w_down;
  const int32_t* ell_rows;    // route of the forward
  const int32_t* dense_rows;
  const int32_t* n_rows;      // device {n_ell, n_dense, over_cap}
  int64_t T, cap;
  int32_t d, F, tile_n, C;
  float l1;
  void* dx;
  float* dw_gate_t;
  float* dw_up_t;
  float* dw_down;
  // workspace
  int32_t* blk_hist;    // [ceil(T/64)][F]
  unsigned long long* blk_mask;  // [ceil(T/64)][F] rows of each 64-row block holding each neuron
  int32_t* neuron_off;  // [F + 1]
  int2* pairs;          // [T * n_t * C] neuron-major {t, slot}
  float2* coef;         // [T][n_t][C] (dg, du) of each stored slot
  float* g_d;           // [cap][F]
  float* u_d;           // [cap][F]
  float* e_d;           // [cap][F] dy_d W_down^T
  void* dg_d;           // [cap][F] dtype
  void* du_d;
  void* h_d;
  float* dx_part;       // [dx_splits][cap][d] fp32 split-K partials of the dense rows' dx
  int32_t dx_splits;
  // light / heavy split of the ELL rows for the dx pass (as in the hybrid forward)
  int32_t* row_total;    // [T]
  int32_t* block_total;  // [ceil(T/256)]
  int32_t* light_rows;   // [T]
  int32_t* heavy_rows;   // [heavy_cap]
  int32_t* split_n;      // [2]
  int32_t* block_heavy;  // [ceil(T/256)]
  int64_t heavy_cap;
  int32_t groups;        // tile ranges per heavy row
  float* dx_hpart;       // [groups][heavy_cap][d] fp32 partial dx of the heavy rows
  int32_t resident;      // lockstep dx pass (set by the launcher): workgroups run at once,
  int64_t blk0;          // and the first row block of this launch
};

// dtype: 0 = fp32, 1 = bf16.  Each returns hipSuccess or the launch error.
hipError_t launch_gate_pack(const PackArgs& a, int dtype, hipStream_t s);
hipError_t launch_fused_updown(const FusedArgs& a, int dtype, hipStream_t s);
hipError_t launch_fused_split(const FusedArgs& a, int dtype, hipStream_t s);
hipError_t launch_gateup(const GateUpArgs& a, int dtype, hipStream_t s);
hipError_t launch_down(const DownArgs& a, int dtype, hipStream_t s);
// Full dense FFN on the 256 x 256 core: transpose w_down into dn.w_down_t,
// gateup256 (all M rows), down256.  dn.h must be g.h.
hipError_t launch_dense256(const GateUpArgs& g, const DownArgs& dn, int dtype, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// After launch_route: split the ELL rows into light rows and at most heavy_cap
// heavy rows (row total > max(2 C, 2 x the mean row total)).
hipError_t launch_route_split(const RouteArgs& a, hipStream_t s);
hipError_t launch_classic_pack(const ClassicArgs& a, int dtype, hipStream_t s);
// out[row(m), :] = round(sum_{s < splits} part[s][m][:]) for m < n_rows (n_rows =
// *n_rows_dev, row(m) = rows[m] or m), summed in ascending s.  d % 4 == 0.
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, const int32_t* n_rows_dev,
                                const int32_t* rows, void* out, int d, int dtype, hipStream_t s);
hipError_t launch_bwd_sparse(const BwdArgs& a, int dtype, hipStream_t s);
hipError_t launch_bwd_dense(const BwdArgs& a, int dtype, hipStream_t s);

// Lockstep launches: how many workgroups of one lockstep kernel (one per CU)
// the current device runs at once; 0 if it cannot be queried.
int lockstep_resident();

}  // namespace twell
