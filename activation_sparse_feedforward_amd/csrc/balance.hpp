// Row balancing of the lockstep kernels (the fused forward and the backward's
// dx pass): which rows each wave of a workgroup takes.
#pragma once
#include "common.hpp"

namespace twell {

// Which rows each wave of a lockstep kernel takes.  Every chunk ends at a
// workgroup barrier, so a chunk lasts as long as the workgroup's busiest wave,
// and the workgroups of an XCD share weight rows through its L2 only while
// they sweep the tiles at the same pace.  Rows are therefore dealt by their
// entry counts over windows of win (<= kWin) consecutive workgroups: every workgroup of
// a window sums the counts of all the window's rows, ranks them (ties by
// position) and deals them snake-wise over the window's W waves (rank r < W to
// wave r, the next W to waves W - 1 .. 0, and so on), so each wave pairs a
// busy row with a quiet one and the window's workgroups carry nearly equal
// work.  Each workgroup computes the same ranking on its own (no
// communication between workgroups) and takes its waves' rows.
//   src[k]: row-list position of the wave's k-th row (>= n_rows: idle)
//   n_blk:  workgroups of the whole grid (every one of them is launched)
//   win:    workgroups per window, 1 .. kWin (uniform over the grid)
//   lds:    2 * kWin * kWaves * TPW ints, 16-byte aligned, that the caller
//           does not touch before its next barrier
//   row_total: per-token sum of the counts, or null (then summed here)
// Every thread of the workgroup must call this (two barriers).
template <int kWaves, int TPW, int kWin>
__device__ __forceinline__ void balance_rows(const int32_t* count, const int32_t* row_total, const int32_t* rows,
                                             int64_t n_rows, int n_t, int64_t blk, int64_t n_blk, int win, int wave,
                                             int* lds, int64_t* src) {
  constexpr int kRpw = kWaves * TPW;  // rows per workgroup
  constexpr int kThreads = kWaves * kWave;
  int* tot = lds;
  int* assign = lds + kWin * kRpw;
  const int64_t win0 = blk / win * win;
  const int nwin = static_cast<int>(min(static_cast<int64_t>(win), n_blk - win0));  // workgroups in the window
  const int nr = nwin * kRpw;
  const int64_t base = win0 * kRpw;
  const int tid = threadIdx.x;
  // row totals: read from row_total[token] where the caller has them, else
  // four threads per row, each summing every fourth tile
  if (row_total) {
    for (int r = tid; r < nr; r += kThreads) {
      const int64_t i_row = base + r;
      tot[r] = i_row < n_rows ? row_total[rows ? static_cast<int64_t>(rows[i_row]) : i_row] : -1;
    }
  } else
  for (int r0 = 0; r0 < nr; r0 += kThreads / 4) {
    const int r = r0 + tid / 4;
    const int64_t i_row = base + r;
    const bool live = r < nr && i_row < n_rows;
    int s = 0;
    if (live) {
      const int64_t t = rows ? static_cast<int64_t>(rows[i_row]) : i_row;
      if ((n_t & 3) == 0) {  // a row of counts is whole 16-byte pieces: four counts per load
        const int4* c4 = reinterpret_cast<const int4*>(count + t * n_t);
        for (int q = tid & 3; q < n_t / 4; q += 4) {
          const int4 v = c4[q];
          s += max(v.x, 0) + max(v.y, 0) + max(v.z, 0) + max(v.w, 0);
        }
      } else {
        for (int b = tid & 3; b < n_t; b += 4) s += max(count[t * n_t + b], 0);
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (r < nr && (tid & 3) == 0) tot[r] = live ? s : -1;
  }
  __syncthreads();
  const int W = nwin * kWaves;
  for (int r = tid; r < nr; r += kThreads) {
    const int tr = tot[r];
    int rank = 0;
    // four totals per LDS read (nr is a multiple of 4, tot 16-byte aligned),
    // several reads in flight: the LDS latency is not paid once per row
#pragma unroll 4
    for (int m = 0; m < nr; m += 4) {
      const int4 tm = *reinterpret_cast<const int4*>(tot + m);
      rank += (tm.x > tr || (tm.x == tr && m < r)) ? 1 : 0;
      rank += (tm.y > tr || (tm.y == tr && m + 1 < r)) ? 1 : 0;
      rank += (tm.z > tr || (tm.z == tr && m + 2 < r)) ? 1 : 0;
      rank += (tm.w > tr || (tm.w == tr && m + 3 < r)) ? 1 : 0;
    }
    const int round = rank / W, within = rank % W;
    assign[((round & 1) ? W - 1 - within : within) * TPW + round] = r;
  }
  __syncthreads();
  const int my = static_cast<int>(blk - win0) * kWaves + wave;
#pragma unroll
  for (int k = 0; k < TPW; ++k) src[k] = base + assign[my * TPW + k];
}

// Workgroups per row-balancing window of the lockstep kernels on a row list
// (the hybrid format's light rows, whose densities spread widely); the plain
// forward (all rows, one density) balances within each workgroup, which costs
// less at its start.
constexpr int kBalanceWindow = 8;

}  // namespace twell
