// Large-tile MFMA GEMM core for gfx950: C[256 x 256] tiles of A . B^T with
// both operands K-contiguous (row-major [rows x K]).
//
//  * 256 threads = 4 waves in a 2 x 2 arrangement; each wave owns a 128 x 128
//    block of C as 4 x 4 blocks of 32x32 MFMA accumulators (256 fp32 per
//    lane, held in AGPRs; one wave per SIMD).  128 columns is one TwELL tile
//    of width 128, so a wave always owns complete rows of the tile it packs.
//  * Operand tiles move global -> LDS with the direct 16-byte loads of gfx950
//    (no VGPR staging): each wave instruction writes 1 KB of LDS = 8 rows of
//    the 128-byte K slice; the lane -> row/chunk assignment applies the same
//    XOR chunk swizzle that the fragment reads use (bank-conflict-free both
//    ways).  Rows past the matrix are clamped to its last row: they only
//    feed output rows/columns that the epilogues discard.
//  * Two LDS stages (2 x 64 KB): the loads of slice k+1 fly while slice k is
//    multiplied; one barrier per slice; the slice body interleaves loads and
//    fragment reads with the MFMAs (see gemm256_mainloop).
//  * Tile order is XCD-aware: consecutive workgroup ids are dealt round-robin
//    to the 8 XCDs, so ids are remapped to give every XCD a contiguous run of
//    tiles, walked in groups of 8 M tiles so that the workgroups resident on
//    one XCD share operand slices in its L2.
#pragma once

#include "common.hpp"

namespace twell {

constexpr int kT256 = 256;                 // BM = BN
constexpr int kStageBytes = 2 * kT256 * 128;  // A + B slice of one stage
constexpr int kLds256 = 2 * kStageBytes;      // two stages

// Tile coordinates of this workgroup (1-D grid of n_mt * n_nt workgroups).
__device__ __forceinline__ void tile_coords_256(int n_mt, int n_nt, int& mt, int& nt) {
  const int nwg = n_mt * n_nt;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * n_nt;
  const int g = pid / per_group;
  const int first = g * kGroupM;
  const int gsize = min(kGroupM, n_mt - first);
  const int in = pid - g * per_group;
  mt = first + in % gsize;
  nt = in / gsize;
}

// One K-contiguous operand: 256 tile rows, each from a matrix row (optionally
// through a row table), ld elements per row.
template <class E>
struct DirectRows {
  const char* ptr[8];  // this lane's source for rounds 0..7 at K slice 0

  // tile row r comes from matrix row row_of(r) = (table ? table[row0 + p(r)] : row0 + p(r)),
  // with row0 + p(r) clamped to nvalid - 1 (nvalid >= 1).  p is the identity, or
  // with lane_cols the permutation inside each 128-row half that puts matrix
  // row 4*l + j at tile row 32*j + l (l < 32, j < 4): used on the B operand,
  // it makes lane l of the wave's accumulator block j hold output column
  // 4*l + j, so every lane holds 4 consecutive columns of its rows.
  __device__ __forceinline__ void init(const void* base, int64_t ld, int64_t row0, int64_t nvalid,
                                       const int32_t* table, bool lane_cols = false) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pc = lane & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = q * 32 + wave * 8 + (lane >> 3);
      const int rp = lane_cols ? ((r & 128) | ((r & 31) << 2) | ((r >> 5) & 3)) : r;
      int64_t gr = row0 + rp;
      gr = gr < nvalid ? gr : nvalid - 1;
      if (table) gr = table[gr];
      const int c = pc ^ lds_swz(r);
      ptr[q] = static_cast<const char*>(base) + gr * ld * E::kBytes + c * 16;
    }
  }
  // Split loader: tile rows [0,64) and [128,192) from `base`, [64,128) and
  // [192,256) from `base2`, both starting at matrix row row0 + (r mod 64) +
  // 64 * (r / 128).  Used by the gate|up GEMM so that each wave's 128 columns
  // hold 64 gate neurons followed by the same 64 up neurons.
  __device__ __forceinline__ void init_split(const void* base, const void* base2, int64_t ld, int64_t row0,
                                             int64_t nvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pc = lane & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = q * 32 + wave * 8 + (lane >> 3);
      const bool second = (r >> 6) & 1;
      int64_t gr = row0 + (r & 63) + 64 * (r >> 7);
      gr = gr < nvalid ? gr : nvalid - 1;
      const int c = pc ^ lds_swz(r);
      ptr[q] = static_cast<const char*>(second ? base2 : base) + gr * ld * E::kBytes + c * 16;
    }
  }
  // One wave instruction (round q) of K slice kt; wave_u is the wave index as a
  // wave-uniform value, so the LDS destination (M0) needs no readfirstlane.
  __device__ __forceinline__ void issue_one(int kt, char* lds_tile, int q, int wave_u) const {
    __builtin_amdgcn_global_load_lds(ptr[q] + static_cast<int64_t>(kt) * 128, lds_tile + (q * 32 + wave_u * 8) * 128,
                                     16, 0, 0);
  }
  __device__ __forceinline__ void issue(int kt, char* lds_tile, int wave_u) const {
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kt, lds_tile, q, wave_u);
  }
};

struct Acc256 {
  f32x16_t c[4][4];
};

__device__ __forceinline__ void read_frag256(Frag<EBf16>& f, const char* lds, int row, int kk, int lane) {
  f.v = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, kk * 2 + (lane >> 5)));
}
__device__ __forceinline__ void read_frag256(Frag<EF32>& f, const char* lds, int row, int kk, int lane) {
  const int c = kk * 4 + (lane >> 5) * 2;
  f.v[0] = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, c));
  f.v[1] = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, c + 1));
}

// nk K slices of 128 bytes.  lds: kLds256 bytes, 16-byte aligned.
//
// With one wave per SIMD, any run of non-MFMA instructions leaves the matrix
// core idle, so the slice body is scheduled by hand (sched_barrier after each
// step pins the order): every MFMA of k-step kk is followed by at most one
// fragment read for k-step kk+1 and, in k-step 0, by one of the 16 direct
// loads of the next slice.  Issued in clumps, the same instructions cost a
// fifth of the loop's cycles.  The last slice re-loads itself into the idle
// stage (keeps the body branch-free); the final vmcnt wait makes sure no
// direct load is still writing LDS when the caller reuses it or the
// workgroup ends.  One barrier per slice, after an explicit wait for this
// wave's direct loads (HIP's __syncthreads would also wait for every load in
// flight).
template <class E>
__device__ __forceinline__ void gemm256_mainloop(const DirectRows<E>& la, const DirectRows<E>& lb, int nk,
                                                 char* lds, Acc256& acc) {
  constexpr int kSteps = 128 / E::kBytes / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int arow = (wave >> 1) * 128 + (lane & 31);
  const int brow = (wave & 1) * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.f;
  if (nk <= 0) return;
  la.issue(0, lds, wave_u);
  lb.issue(0, lds + kT256 * 128, wave_u);
  for (int kt = 0; kt < nk; ++kt) {
    const int kl = kt + 1 < nk ? kt + 1 : kt;
    const char* A = lds + (kt & 1) * kStageBytes;
    const char* B = A + kT256 * 128;
    char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    Frag<E> a[2][4], b[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) read_frag256(a[0][i], A, arow + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) read_frag256(b[0][j], B, brow + j * 32, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
      const int cb = kk & 1;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma_k16(acc.c[m >> 2][m & 3], a[cb][m >> 2], b[cb][m & 3]);
        if (kk + 1 < kSteps && m < 8) {
          if (m < 4)
            read_frag256(a[cb ^ 1][m], A, arow + m * 32, kk + 1, lane);
          else
            read_frag256(b[cb ^ 1][m - 4], B, brow + (m - 4) * 32, kk + 1, lane);
        }
        if (kk == 0) {
          if (m < 8)
            la.issue_one(kl, nxt, m, wave_u);
          else
            lb.issue_one(kl, nxt + kT256 * 128, m - 8, wave_u);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace twell
