// MFMA GEMM core for gfx950: a 256-thread workgroup computes a 256 x BN fp32
// tile of C = A * B^T-style products, staging 128-byte K slices of both
// operands through LDS.  Four waves; wave w owns rows [64w, 64w + 64) and all
// BN columns, i.e. 2 x (BN/32) blocks of 32x32 accumulators.  Owning whole
// rows lets the TwELL epilogue compact a full T_n-wide tile from registers.
#pragma once

#include "common.hpp"

namespace twell {

constexpr int kBM = 256;
constexpr int kThreads = 256;
constexpr uint32_t kNoRow = 0xffffffffu;

// ---------------------------------------------------------------------------
// Operand with K contiguous: R rows of a row-major matrix (ld elements per row).
// Each thread moves R/32 16-byte chunks per 128-byte K slice.  Row indices may
// go through an indirection table (gathered rows); rows past `nvalid` read as 0.
// ---------------------------------------------------------------------------
template <class E, int R>
struct KRowLoader {
  static constexpr int kPer = R / 32;
  static constexpr int kSliceElems = 128 / E::kBytes;
  const char* base;
  uint32_t row_off[kPer];  // element offset of the row start, or kNoRow
  int chunk;
  u32x4_t regs[kPer];

  // row r of the tile is matrix row row0 + r (or rows[row0 + r] when rows != nullptr)
  __device__ __forceinline__ void init(const void* ptr, int64_t ld, int64_t row0, int64_t nvalid,
                                       const int32_t* rows) {
    base = static_cast<const char*>(ptr);
    const int tid = threadIdx.x;
    chunk = tid & 7;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      int64_t r = row0 + (tid >> 3) + 32 * p;
      if (r < nvalid) {
        int64_t mr = rows ? static_cast<int64_t>(rows[r]) : r;
        row_off[p] = static_cast<uint32_t>(mr * ld);
      } else {
        row_off[p] = kNoRow;
      }
    }
  }
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      if (row_off[p] != kNoRow) {
        const char* a = base + (static_cast<uint64_t>(row_off[p]) + static_cast<uint64_t>(kt) * kSliceElems) *
                                   E::kBytes + chunk * 16;
        regs[p] = *reinterpret_cast<const u32x4_t*>(a);
      } else {
        regs[p] = u32x4_t{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int row_base) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      int row = row_base + (tid >> 3) + 32 * p;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(row, chunk)) = regs[p];
    }
  }
};

// ---------------------------------------------------------------------------
// Operand with MN contiguous: the matrix is stored [K x MN] row-major (ld = MN
// elements) and the tile is R columns (mn0 ..) by one 128-byte K slice.  Each
// thread loads four K rows of one 16-byte MN chunk and writes them transposed
// into the K-contiguous LDS layout.  K rows may go through an indirection
// table (gathered rows); K rows past `k_total` and columns past `mn_total`
// read as 0 (mn_total must be a multiple of 16 bytes' worth of elements).
// ---------------------------------------------------------------------------
template <class E, int R>
struct MNColLoader {
  static constexpr int kSliceElems = 128 / E::kBytes;        // K rows per slice
  static constexpr int kMnChunks = R / E::kPer16B;           // 16-byte chunks across the tile
  static constexpr int kUnits = kMnChunks * (kSliceElems / 4);
  static constexpr int kPer = kUnits / kThreads;
  static_assert(kUnits % kThreads == 0, "tile shape");
  const char* base;
  int64_t ld;
  int64_t k_total;
  int64_t mn0;
  int64_t mn_total;
  const int32_t* rows;
  u32x4_t regs[kPer][4];

  __device__ __forceinline__ void init(const void* ptr, int64_t ld_, int64_t mn0_, int64_t mn_total_,
                                       int64_t k_total_, const int32_t* rows_ = nullptr) {
    base = static_cast<const char*>(ptr);
    ld = ld_;
    mn0 = mn0_;
    mn_total = mn_total_;
    k_total = k_total_;
    rows = rows_;
  }
  __device__ __forceinline__ void load(int kt) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kThreads;
      const int mnc = u % kMnChunks, kq = u / kMnChunks;
      const bool col_ok = mn0 + mnc * E::kPer16B < mn_total;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t k = static_cast<int64_t>(kt) * kSliceElems + kq * 4 + i;
        if (col_ok && k < k_total) {
          const int64_t kr = rows ? static_cast<int64_t>(rows[k]) : k;
          const char* a = base + (kr * ld + mn0 + mnc * E::kPer16B) * E::kBytes;
          regs[p][i] = *reinterpret_cast<const u32x4_t*>(a);
        } else {
          regs[p][i] = u32x4_t{0, 0, 0, 0};
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int row_base) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kThreads;
      const int mnc = u % kMnChunks, kq = u / kMnChunks;
      if constexpr (E::kBytes == 2) {
        // four K rows x eight bf16 columns -> eight 8-byte K runs, one per column
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t lo, hi;
          if ((e & 1) == 0) {
            lo = (regs[p][0][w] & 0xffffu) | (regs[p][1][w] << 16);
            hi = (regs[p][2][w] & 0xffffu) | (regs[p][3][w] << 16);
          } else {
            lo = (regs[p][0][w] >> 16) | (regs[p][1][w] & 0xffff0000u);
            hi = (regs[p][2][w] >> 16) | (regs[p][3][w] & 0xffff0000u);
          }
          const int row = row_base + mnc * 8 + e;
          *reinterpret_cast<u32x2_t*>(lds + lds_off(row, kq >> 1) + ((kq & 1) << 3)) = u32x2_t{lo, hi};
        }
      } else {
        // four K rows x four fp32 columns -> four 16-byte K runs, one per column
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = row_base + mnc * 4 + e;
          *reinterpret_cast<u32x4_t*>(lds + lds_off(row, kq)) =
              u32x4_t{regs[p][0][e], regs[p][1][e], regs[p][2][e], regs[p][3][e]};
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Fragment reads (see mfma_k16 for the lane -> k assignment).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void read_frag(Frag<EBf16>& f, const char* lds, int row, int kk, int lane) {
  f.v = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, kk * 2 + (lane >> 5)));
}
__device__ __forceinline__ void read_frag(Frag<EF32>& f, const char* lds, int row, int kk, int lane) {
  const int c = kk * 4 + (lane >> 5) * 2;
  f.v[0] = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, c));
  f.v[1] = *reinterpret_cast<const u32x4_t*>(lds + lds_off(row, c + 1));
}

template <int BN>
struct Acc {
  static constexpr int kWN = BN / 32;
  f32x16_t c[2][kWN];
};

// ---------------------------------------------------------------------------
// Main loop: nk K slices.  Shared-memory layout: A tile (256 rows) then B tile
// (BN rows), 128 bytes per row.  Register prefetch of slice kt+1 overlaps the
// MFMAs of slice kt.
// ---------------------------------------------------------------------------
template <class E, int BN, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* lds, Acc<BN>& acc,
                                              bool accumulate = false) {
  constexpr int kWN = BN / 32;
  constexpr int kSteps = 128 / E::kBytes / 16;
  char* ldsA = lds;
  char* ldsB = lds + kBM * 128;
  const int lane = threadIdx.x & 63;
  const int wrow = (threadIdx.x >> 6) * 64;
  if (!accumulate) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kWN; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc.c[mb][nb][r] = 0.f;
  }
  if (nk <= 0) return;
  la.load(0);
  lb.load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    la.store(ldsA, 0);
    lb.store(ldsB, 0);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
      Frag<E> a[2], b[kWN];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) read_frag(a[mb], ldsA, wrow + mb * 32 + (lane & 31), kk, lane);
#pragma unroll
      for (int nb = 0; nb < kWN; ++nb) read_frag(b[nb], ldsB, nb * 32 + (lane & 31), kk, lane);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < kWN; ++nb) mfma_k16(acc.c[mb][nb], a[mb], b[nb]);
    }
  }
}

}  // namespace twell
