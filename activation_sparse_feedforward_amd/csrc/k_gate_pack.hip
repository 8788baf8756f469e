// Gate GEMM with a ReLU + TwELL-packing epilogue, one dispatch.
//
// Follows the TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA
// kernels...", section "¿Qué hace distinto a TwELL frente a ELL clásico?"):
// the sparse format is produced inside the epilogue of the gate matmul, the
// activation columns are cut into tiles equal to the matmul's N tile, and the
// non-zeros are packed locally per tile.  Here every wave owns complete rows
// of one TwELL tile in its MFMA accumulators, so each (row, tile) is compacted
// on chip: a wavefront ballot per 32-column block gives the non-zero mask of
// two rows at once, and the masks give every non-zero its slot in ascending
// column order -- no atomics and no dense store of ReLU(g); the compact
// records leave with wide stores.  bf16 with 16 slots (the 2B-class format)
// stages the rounded rows in LDS and lets each lane pack one row
// (pack_epilogue_rows); other formats compact straight from the accumulator
// registers (pack_epilogue_lc, pack_epilogue).
//
// T_n = 128 uses the 256 x 256 direct-to-LDS core (gemm256.hpp); T_n = 64 the
// 256 x 64 register-staged core (gemm_core.hpp); batches of at most 64 tokens
// (bf16, T_n = 128) a kernel that streams W_gate once (gate_pack_small_kernel).
#include <algorithm>

#include "gemm256.hpp"
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

// Compact one wave's accumulators (rows wrow0 .. wrow0 + 32*MB, TwELL tile b of
// width 32*KWN) into TwELL.  Register r of a 32x32 block holds, in lanes 0-31,
// 32 columns of one row and, in lanes 32-63, the same columns of the row 4
// below, so one 64-bit ballot per (register, 32-column block) is the non-zero
// mask of two rows.  Almost all of the work is scalar: an all-zero block is
// skipped on a uniform branch, slot = mbcnt(mask) + running count of the row
// (the running counts are SGPR popcounts), per-row counts are parked in one
// VGPR (lane i = row i), and only the non-zeros are rounded and stored.
//
// A value is a non-zero iff its stored (dtype-rounded) value is: for bf16,
// round-to-nearest-even of a positive fp32 u is non-zero iff bits(u) >= 0x8001
// (below that the value rounds to +0), so one signed integer compare on the
// fp32 bits decides it (negative values and -0 have the sign bit set).
//
// The records of 32 rows at a time are assembled in this wave's LDS scratch
// (zeroed first, so unused slots need no stores) and leave with 16-byte
// stores.  wlds: pack_scratch_bytes(C, sizeof(dtype)) bytes, 16-byte aligned.
template <class E, int MB, int KWN, bool DBG>
__device__ __forceinline__ void pack_epilogue(const PackArgs& p, const f32x16_t (&acc)[MB][KWN], int64_t wrow0,
                                              int b, char* wlds, uint32_t& ovf, uint32_t& nnz) {
  constexpr int kTn = 32 * KWN;
  constexpr int kNzMin = E::kBytes == 2 ? 0x8001 : 1;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, li = lane & 31;
  const int n_t = p.F / kTn;
  const int C = p.C;
  const int idx_bytes = C, val_bytes = C * E::kBytes;
  uint8_t* l_idx = reinterpret_cast<uint8_t*>(wlds);
  char* l_val = wlds + 32 * idx_bytes;
  const int rec_words = 32 * (idx_bytes + val_bytes) / 4;
  // copy pieces: 16 bytes when every record is a multiple of 16 bytes, else 4, else 1
  const int piece = (C % 16) == 0 ? 16 : ((C % 4) == 0 ? 4 : 1);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    for (int i = lane; i < rec_words; i += 64) reinterpret_cast<uint32_t*>(wlds)[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t row0 = wrow0 + mb * 32;
    int cnt_v = 0;  // lane i < 32: count of row row0 + i
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ra = 8 * (r >> 2) + (r & 3);  // row of lanes 0-31; lanes 32-63 hold row ra + 4
      const int rr = ra + 4 * half;
      int pre_a = 0, pre_b = 0;
#pragma unroll
      for (int nb = 0; nb < KWN; ++nb) {
        const uint32_t u = __float_as_uint(acc[mb][nb][r]);
        const bool nz = static_cast<int>(u) >= kNzMin;
        if constexpr (DBG) {
          const int64_t row = row0 + rr;
          if (row < p.T)
            store_bits<E>(p.gate_dbg, row * p.F + static_cast<int64_t>(b) * kTn + nb * 32 + li,
                          nz ? round_store<E>(__uint_as_float(u)).bits : 0u);
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(nz);
        if (m != 0) {
          const uint32_t mlo = static_cast<uint32_t>(m), mhi = static_cast<uint32_t>(m >> 32);
          const int plo = __popc(mlo), phi = __popc(mhi);
          const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u)));
          const int s = below + (half ? pre_b - plo : pre_a);
          if (nz && s < C) {
            l_idx[rr * idx_bytes + s] = static_cast<uint8_t>(nb * 32 + li);
            const uint32_t bits = round_store<E>(__uint_as_float(u)).bits;
            if constexpr (E::kBytes == 2)
              reinterpret_cast<uint16_t*>(l_val + rr * val_bytes)[s] = static_cast<uint16_t>(bits);
            else
              reinterpret_cast<uint32_t*>(l_val + rr * val_bytes)[s] = bits;
          }
          pre_a += plo;
          pre_b += phi;
        }
      }
      cnt_v = lane == ra ? pre_a : (lane == ra + 4 ? pre_b : cnt_v);
      if (row0 + ra < p.T) {
        ovf += pre_a > C ? 1u : 0u;
        nnz += static_cast<uint32_t>(pre_a);
      }
      if (row0 + ra + 4 < p.T) {
        ovf += pre_b > C ? 1u : 0u;
        nnz += static_cast<uint32_t>(pre_b);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // write the 32 records out: counts, then index and value pieces
    if (lane < 32 && row0 + lane < p.T) p.count[(row0 + lane) * n_t + b] = cnt_v;
    const int ip = idx_bytes / piece, vp = val_bytes / piece;  // pieces per row
    for (int w = lane; w < 32 * (ip + vp); w += 64) {
      const int rw = w / (ip + vp), k = w - rw * (ip + vp);
      const int64_t row = row0 + rw;
      if (row >= p.T) continue;
      const int64_t rt = row * n_t + b;
      const char* src;
      char* dst;
      if (k < ip) {
        src = reinterpret_cast<const char*>(l_idx) + rw * idx_bytes + k * piece;
        dst = reinterpret_cast<char*>(p.idx) + rt * idx_bytes + k * piece;
      } else {
        src = l_val + rw * val_bytes + (k - ip) * piece;
        dst = static_cast<char*>(p.val) + rt * val_bytes + (k - ip) * piece;
      }
      if (piece == 16)
        *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
      else if (piece == 4)
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
      else
        *dst = *src;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Lane-column variant for a wave tile of 128 rows x one TwELL tile of 128
// columns whose B operand was loaded with DirectRows' lane_cols permutation:
// lane l of accumulator block j holds tile column 4*l + j, so each lane holds 4
// consecutive columns of a row, and a row's ascending column order is lane
// order, then j.  One register index r covers 2 rows x 128 columns (lanes 0-31:
// row ra, lanes 32-63: row ra + 4).
//
// With one wave per SIMD this code is bound by instruction issue, so the
// common case is short and branch-free.  "Stored value is non-zero" is a
// signed compare of the fp32 bits, so per lane the largest and the second
// largest bit pattern of its four values tell whether it holds any, and
// whether it holds two or more, non-zeros.  Registers with no non-zero at all
// are skipped.  When no lane holds two or more (one uniform test), a row's
// count is the popcount of the "lane has a non-zero" mask over its half, a
// non-zero's slot is that mask's exclusive prefix (mbcnt), its value is the
// lane's largest, and every lane writes one index byte and one value, lanes
// with nothing to store (or past C) into a private dummy slot.  Registers
// where some lane holds two or more non-zeros take a general path: the prefix
// over the per-lane counts c (0..4) is built from the ballots of c >= k,
// k = 1..4.
// Records are assembled in LDS exactly as in pack_epilogue; the counts go
// into lane i < 32 of one register (row i) with v_writelane.  The statistics
// (overflowing tiles, non-zeros) are computed from the final counts, and only
// when asked.  kC > 0 fixes C at compile time (record offsets become
// immediates); 0 reads p.C.
// wlds: pack_lc_scratch_bytes(C, sizeof(dtype)) bytes, 16-byte aligned.
template <class E, bool DBG, int kC>
__device__ __forceinline__ void pack_epilogue_lc(const PackArgs& p, const f32x16_t (&acc)[4][4], int64_t wrow0,
                                                 int b, char* wlds, uint32_t& ovf, uint32_t& nnz) {
  constexpr int kNzMin = E::kBytes == 2 ? 0x8001 : 1;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, li = lane & 31;
  const int n_t = p.F / 128;
  const int C = kC > 0 ? kC : p.C;
  const int idx_bytes = C, val_bytes = C * E::kBytes;
  uint8_t* l_idx = reinterpret_cast<uint8_t*>(wlds);
  char* l_val = wlds + 32 * idx_bytes;
  const int rec_bytes = 32 * (idx_bytes + val_bytes);  // a multiple of 16
  uint8_t* dummy_idx = reinterpret_cast<uint8_t*>(wlds + rec_bytes) + lane;
  char* dummy_val = wlds + rec_bytes + 64 + lane * E::kBytes;
  const uint32_t half_mask = half ? 0xffffffffu : 0u;
  const int piece = (C % 16) == 0 ? 16 : ((C % 4) == 0 ? 4 : 1);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    for (int i = lane; i < rec_bytes / 16; i += 64) reinterpret_cast<u32x4_t*>(wlds)[i] = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t row0 = wrow0 + mb * 32;
    int cnt_v = 0;  // lane i < 32: count of row row0 + i
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ra = 8 * (r >> 2) + (r & 3);
      const int rr = ra + 4 * half;
      int u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = __float_as_int(acc[mb][j][r]);
      if constexpr (DBG) {
        const int64_t row = row0 + rr;
        if (row < p.T)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store_bits<E>(p.gate_dbg, row * p.F + static_cast<int64_t>(b) * 128 + 4 * li + j,
                          u[j] >= kNzMin ? round_store<E>(__int_as_float(u[j])).bits : 0u);
      }
      // The test "stored value is non-zero" is a signed compare of the fp32
      // bits, so the largest and second largest bit patterns of the lane's four
      // values say whether it holds one, or two or more, non-zeros.
      const int top3 = max(max(u[0], u[1]), u[2]);
      const int big = max(top3, u[3]);
      const uint64_t any = __builtin_amdgcn_ballot_w64(big >= kNzMin);
      if (any == 0) continue;
      const int med3 = max(min(u[0], u[1]), min(max(u[0], u[1]), u[2]));
      const int second = max(med3, min(top3, u[3]));
      const uint64_t two = __builtin_amdgcn_ballot_w64(second >= kNzMin);
      const uint32_t lo1 = static_cast<uint32_t>(any), hi1 = static_cast<uint32_t>(any >> 32);
      const int excl1 = static_cast<int>(__builtin_amdgcn_mbcnt_hi(hi1, __builtin_amdgcn_mbcnt_lo(lo1, 0u))) -
                        static_cast<int>(static_cast<uint32_t>(__popc(lo1)) & half_mask);
      if (__builtin_expect(two == 0, 1)) {
        // at most one non-zero per lane, and it is the largest value
        const int pre_a = __popc(lo1), pre_b = __popc(hi1);
        asm("v_writelane_b32 %0, %1, %2" : "+v"(cnt_v) : "s"(pre_a), "i"(ra));
        asm("v_writelane_b32 %0, %1, %2" : "+v"(cnt_v) : "s"(pre_b), "i"(ra + 4));
        const int jj = u[0] >= kNzMin ? 0 : (u[1] >= kNzMin ? 1 : (u[2] >= kNzMin ? 2 : 3));
        const bool ok = big >= kNzMin && excl1 < C;
        uint8_t* ia = ok ? l_idx + rr * idx_bytes + excl1 : dummy_idx;
        char* va = ok ? l_val + rr * val_bytes + excl1 * E::kBytes : dummy_val;
        *ia = static_cast<uint8_t>(4 * li + jj);
        const uint32_t vb = round_store<E>(__int_as_float(big)).bits;
        if constexpr (E::kBytes == 2)
          *reinterpret_cast<uint16_t*>(va) = static_cast<uint16_t>(vb);
        else
          *reinterpret_cast<uint32_t*>(va) = vb;
      } else {
        bool nz[4];
        int pre_a = 0, pre_b = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          nz[j] = u[j] >= kNzMin;
          const uint64_t mj = __builtin_amdgcn_ballot_w64(nz[j]);
          pre_a += __popc(static_cast<uint32_t>(mj));
          pre_b += __popc(static_cast<uint32_t>(mj >> 32));
        }
        asm("v_writelane_b32 %0, %1, %2" : "+v"(cnt_v) : "s"(pre_a), "i"(ra));
        asm("v_writelane_b32 %0, %1, %2" : "+v"(cnt_v) : "s"(pre_b), "i"(ra + 4));
        const int bits = (nz[0] ? 1 : 0) | (nz[1] ? 2 : 0) | (nz[2] ? 4 : 0) | (nz[3] ? 8 : 0);
        const int c = __popc(bits);
        int excl = excl1;
#pragma unroll
        for (int k = 2; k <= 4; ++k) {
          const uint64_t mk = __builtin_amdgcn_ballot_w64(c >= k);
          const uint32_t lo = static_cast<uint32_t>(mk), hi = static_cast<uint32_t>(mk >> 32);
          excl += static_cast<int>(__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u))) -
                  static_cast<int>(static_cast<uint32_t>(__popc(lo)) & half_mask);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (nz[j]) {
            const int s = excl + __popc(bits & ((1 << j) - 1));
            if (s < C) {
              l_idx[rr * idx_bytes + s] = static_cast<uint8_t>(4 * li + j);
              const uint32_t vb = round_store<E>(__int_as_float(u[j])).bits;
              if constexpr (E::kBytes == 2)
                reinterpret_cast<uint16_t*>(l_val + rr * val_bytes)[s] = static_cast<uint16_t>(vb);
              else
                reinterpret_cast<uint32_t*>(l_val + rr * val_bytes)[s] = vb;
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool row_ok = lane < 32 && row0 + lane < p.T;
    if (p.stats) {
      const int cv = row_ok ? cnt_v : 0;
      ovf += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(cv > C)));
      int sum = cv;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      nnz += static_cast<uint32_t>(__shfl(sum, 0));
    }
    if (row_ok) p.count[(row0 + lane) * n_t + b] = cnt_v;
    const int ip = idx_bytes / piece, vp = val_bytes / piece;
    for (int w = lane; w < 32 * (ip + vp); w += 64) {
      const int rw = w / (ip + vp), k = w - rw * (ip + vp);
      const int64_t row = row0 + rw;
      if (row >= p.T) continue;
      const int64_t rt = row * n_t + b;
      const char* src;
      char* dst;
      if (k < ip) {
        src = reinterpret_cast<const char*>(l_idx) + rw * idx_bytes + k * piece;
        dst = reinterpret_cast<char*>(p.idx) + rt * idx_bytes + k * piece;
      } else {
        src = l_val + rw * val_bytes + (k - ip) * piece;
        dst = static_cast<char*>(p.val) + rt * val_bytes + (k - ip) * piece;
      }
      if (piece == 16)
        *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(src);
      else if (piece == 4)
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
      else
        *dst = *src;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Row-staged variant for bf16 and C = 16, for a wave tile of 128 rows x one
// TwELL tile of 128 columns whose B operand was loaded in natural order (lane
// l of accumulator block j holds tile column 32 j + l).  The wave's rows are
// handled in two halves of 64:
//  1. per accumulator register (two rows x 32 columns per block), ReLU(g) is
//     rounded to bf16 with the packed conversion (round to nearest even) and
//     written to this wave's LDS scratch as row-major rows; one ballot per
//     32-column block is the non-zero mask of those columns of the two rows,
//     in ascending column order, and lane i collects (v_writelane) the four
//     mask words of row i;
//  2. lane i then owns row i: its count is the popcount of its mask, and it
//     takes its first C non-zeros in ascending column order by repeatedly
//     clearing the lowest set bit, reading each value back from the row in
//     LDS and placing index and value into a 48-byte record held in registers,
//     which leaves with three 16-byte stores.
// A stored value is non-zero iff the fp32 bits are >= 0x8001 (signed), so the
// masks come from the accumulator bits, clamped at 0 (the ReLU) as integers.
// (Only masked positions are read back, so the clamp matters only for the
// debug copy of the rows; without it the compiler copies the accumulators out
// early and spills nine registers per lane, 19 MB of scratch traffic per call.)
// There are no per-register branches and no cross-lane slot arithmetic.
// wlds: kRowsScratch bytes, 16-byte aligned.
constexpr int kRowStride = 272;                      // 256 B of values + 16 B so rows start on different banks
constexpr int kRowsScratch = 64 * kRowStride;        // one half (64 rows) per wave

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2v));
}

template <bool DBG>
__device__ __forceinline__ void pack_epilogue_rows(const PackArgs& p, const f32x16_t (&acc)[4][4], int64_t wrow0,
                                                   int b, char* wlds, uint32_t& ovf, uint32_t& nnz) {
  constexpr int C = 16;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, li = lane & 31;
  const int n_t = p.F / 128;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    uint32_t mk[4] = {0u, 0u, 0u, 0u};  // lane i: non-zero mask of row i of this half, columns 32 w ..
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int mb = 2 * hb + m2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ra = m2 * 32 + 8 * (r >> 2) + (r & 3);  // row of lanes 0-31 in the half; lanes 32-63: ra + 4
        int u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u[j] = max(__float_as_int(acc[mb][j][r]), 0);
        }
        uint16_t* rowp = reinterpret_cast<uint16_t*>(wlds + (ra + 4 * half) * kRowStride);
        const uint32_t p01 = cvt_pk_bf16(__int_as_float(u[0]), __int_as_float(u[1]));
        const uint32_t p23 = cvt_pk_bf16(__int_as_float(u[2]), __int_as_float(u[3]));
        rowp[li] = static_cast<uint16_t>(p01);
        rowp[32 + li] = static_cast<uint16_t>(p01 >> 16);
        rowp[64 + li] = static_cast<uint16_t>(p23);
        rowp[96 + li] = static_cast<uint16_t>(p23 >> 16);
        uint64_t m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = __builtin_amdgcn_ballot_w64(u[j] >= 0x8001);
        // lane ra takes row ra's mask words, lane ra + 4 those of row ra + 4.
        // A VALU read of an SGPR that a VALU compare has just written needs two
        // wait states, which the compiler cannot insert inside the asm.
        asm("s_nop 1\n\t"
            "v_writelane_b32 %0, %4, %12\n\tv_writelane_b32 %0, %5, %13\n\t"
            "v_writelane_b32 %1, %6, %12\n\tv_writelane_b32 %1, %7, %13\n\t"
            "v_writelane_b32 %2, %8, %12\n\tv_writelane_b32 %2, %9, %13\n\t"
            "v_writelane_b32 %3, %10, %12\n\tv_writelane_b32 %3, %11, %13"
            : "+v"(mk[0]), "+v"(mk[1]), "+v"(mk[2]), "+v"(mk[3])
            : "s"(static_cast<uint32_t>(m[0])), "s"(static_cast<uint32_t>(m[0] >> 32)),
              "s"(static_cast<uint32_t>(m[1])), "s"(static_cast<uint32_t>(m[1] >> 32)),
              "s"(static_cast<uint32_t>(m[2])), "s"(static_cast<uint32_t>(m[2] >> 32)),
              "s"(static_cast<uint32_t>(m[3])), "s"(static_cast<uint32_t>(m[3] >> 32)), "i"(ra), "i"(ra + 4));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t row = wrow0 + hb * 64 + lane;
    const bool row_ok = row < p.T;
    const uint16_t* myrow = reinterpret_cast<const uint16_t*>(wlds + lane * kRowStride);
    if constexpr (DBG) {
      if (row_ok) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(myrow);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.gate_dbg) + (row * p.F + b * 128) * 2);
#pragma unroll
        for (int c = 0; c < 16; ++c) dst[c] = src[c];
      }
    }
    const int cnt = __builtin_popcount(mk[0]) + __builtin_popcount(mk[1]) + __builtin_popcount(mk[2]) +
                    __builtin_popcount(mk[3]);
    uint32_t ri[4] = {0u, 0u, 0u, 0u};                  // C index bytes
    uint32_t rv[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // C bf16 values
#pragma unroll
    for (int s = 0; s < C; ++s) {
      if (__builtin_amdgcn_ballot_w64(s < cnt) == 0) break;  // uniform: no row has another non-zero
      if (s < cnt) {
        const bool z0 = mk[0] == 0u, z1 = mk[1] == 0u, z2 = mk[2] == 0u;
        const uint32_t w = !z0 ? mk[0] : (!z1 ? mk[1] : (!z2 ? mk[2] : mk[3]));
        const int col = (!z0 ? 0 : (!z1 ? 32 : (!z2 ? 64 : 96))) + __builtin_ctz(w);
        const uint32_t wc = w & (w - 1u);
        if (!z0) mk[0] = wc;
        else if (!z1) mk[1] = wc;
        else if (!z2) mk[2] = wc;
        else mk[3] = wc;
        ri[s >> 2] |= static_cast<uint32_t>(col) << (8 * (s & 3));
        rv[s >> 1] |= static_cast<uint32_t>(myrow[col]) << (16 * (s & 1));
      }
    }
    if (row_ok) {
      const int64_t rt = row * n_t + b;
      p.count[rt] = cnt;
      *reinterpret_cast<u32x4_t*>(p.idx + rt * C) = u32x4_t{ri[0], ri[1], ri[2], ri[3]};
      u32x4_t* vd = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.val) + rt * C * 2);
      vd[0] = u32x4_t{rv[0], rv[1], rv[2], rv[3]};
      vd[1] = u32x4_t{rv[4], rv[5], rv[6], rv[7]};
    }
    if (p.stats) {
      const int cv = row_ok ? cnt : 0;
      ovf += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(cv > C)));
      nnz += static_cast<uint32_t>(wave_last(wave_incl_scan(cv)));
    }
    __builtin_amdgcn_wave_barrier();  // all rows read before the next half overwrites them
  }
}

// Bytes of LDS scratch one wave's epilogue needs.
__host__ __device__ constexpr int pack_scratch_bytes(int C, int eb) { return ((32 * C * (1 + eb)) + 15) & ~15; }
// The lane-column epilogue adds 64 dummy index bytes and 64 dummy values (one per lane).
__host__ __device__ constexpr int pack_lc_scratch_bytes(int C, int eb) { return pack_scratch_bytes(C, eb) + 64 + 64 * eb; }

// ovf / nnz are wave-uniform (they are built from ballot popcounts), so lane 0
// publishes the wave's totals.
__device__ __forceinline__ void pack_stats(const PackArgs& p, uint32_t ovf, uint32_t nnz) {
  if (!p.stats) return;
  if ((threadIdx.x & 63) == 0) {
    if (ovf) atomicAdd(p.stats + 0, static_cast<unsigned long long>(ovf));
    if (nnz) atomicAdd(p.stats + 1, static_cast<unsigned long long>(nnz));
  }
}

// T_n = 128: 256 x 256 workgroup tile (two TwELL tiles); wave w owns rows
// [128*(w/2), +128) and TwELL tile 2*nt + (w%2).
template <class E, bool DBG, int kC>
__global__ __launch_bounds__(256, 1) void gate_pack256_kernel(PackArgs p) {
  // bf16 with C = 16 takes the row-staged epilogue (natural column order on
  // the B operand); other cases the lane-column one
  constexpr bool kRows = E::kBytes == 2 && kC == 16;
  extern __shared__ __align__(16) char lds[];
  const int n_mt = static_cast<int>((p.T + kT256 - 1) / kT256);
  const int n_nt = (p.F + kT256 - 1) / kT256;
  int mt, nt;
  tile_coords_256(n_mt, n_nt, mt, nt);
  const int64_t m0 = static_cast<int64_t>(mt) * kT256;
  const int64_t n0 = static_cast<int64_t>(nt) * kT256;
  DirectRows<E> la, lb;
  la.init(p.x, p.d, m0, p.T, nullptr);
  lb.init(p.w_gate_t, p.d, n0, p.F, nullptr, /*lane_cols=*/!kRows);
  Acc256 acc;
  gemm256_mainloop<E>(la, lb, p.d / (128 / E::kBytes), lds, acc);
  const int wave = threadIdx.x >> 6;
  const int b = static_cast<int>((n0 >> 7) + (wave & 1));
  uint32_t ovf = 0, nnz = 0;
  __syncthreads();  // every wave is done with the operand stages: reuse them as epilogue scratch
  if constexpr (kRows) {
    if (b < p.F / 128) pack_epilogue_rows<DBG>(p, acc.c, m0 + (wave >> 1) * 128, b, lds + wave * kRowsScratch, ovf, nnz);
  } else {
    char* wlds = lds + wave * pack_lc_scratch_bytes(kC > 0 ? kC : p.C, E::kBytes);
    if (b < p.F / 128) pack_epilogue_lc<E, DBG, kC>(p, acc.c, m0 + (wave >> 1) * 128, b, wlds, ovf, nnz);
  }
  pack_stats(p, ovf, nnz);
}

// T_n = 64: 256 x 64 workgroup tile (one TwELL tile); wave w owns rows [64w, +64).
template <class E, bool DBG>
__global__ __launch_bounds__(kThreads, 2) void gate_pack64_kernel(PackArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  KRowLoader<E, kBM> la;
  KRowLoader<E, 64> lb;
  la.init(p.x, p.d, m0, p.T, nullptr);
  lb.init(p.w_gate_t, p.d, static_cast<int64_t>(b) * 64, p.F, nullptr);
  Acc<64> acc;
  gemm_mainloop<E, 64>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);
  uint32_t ovf = 0, nnz = 0;
  __syncthreads();
  char* wlds = lds + (threadIdx.x >> 6) * pack_scratch_bytes(p.C, E::kBytes);
  pack_epilogue<E, 2, 2, DBG>(p, acc.c, m0 + (threadIdx.x >> 6) * 64, b, wlds, ovf, nnz);
  pack_stats(p, ovf, nnz);
}

template <class E, bool DBG, int kC>
static hipError_t launch_pack256_c(const PackArgs& a, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gate_pack256_kernel<E, DBG, kC>), hipFuncAttributeMaxDynamicSharedMemorySize,
      kLds256);
  if (attr != hipSuccess) return attr;
  const unsigned n_mt = static_cast<unsigned>((a.T + kT256 - 1) / kT256);
  const unsigned n_nt = static_cast<unsigned>((a.F + kT256 - 1) / kT256);
  hipLaunchKernelGGL((gate_pack256_kernel<E, DBG, kC>), dim3(n_mt * n_nt), dim3(256), kLds256, s, a);
  return hipGetLastError();
}

template <class E, bool DBG>
static hipError_t launch_pack256_t(const PackArgs& a, hipStream_t s) {
  // 4 waves' epilogue scratch must fit in the operand stages it reuses
  static_assert(4 * pack_lc_scratch_bytes(128, 4) <= kLds256, "pack scratch exceeds the GEMM stages");
  static_assert(4 * kRowsScratch <= kLds256, "row scratch exceeds the GEMM stages");
  return a.C == 16 ? launch_pack256_c<E, DBG, 16>(a, s) : launch_pack256_c<E, DBG, 0>(a, s);
}

template <class E, bool DBG>
static hipError_t launch_pack64_t(const PackArgs& a, hipStream_t s) {
  dim3 grid(a.F / 64, static_cast<unsigned>((a.T + kBM - 1) / kBM));
  const size_t lds = std::max<size_t>((kBM + 64) * 128, 4 * pack_scratch_bytes(a.C, E::kBytes));
  hipLaunchKernelGGL((gate_pack64_kernel<E, DBG>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// Small and mid-size batches (bf16, T_n = 128; see use_small): the work is
// mostly reading W_gate, so the tiling is turned around.  One workgroup per
// TwELL tile (128 neurons) and block of up to 128 tokens (one block up to 64
// tokens); the neurons are the MFMA's M side and the tokens its N side.  With only F/128
// workgroups each CU must stream its tile's 128 weight rows fast, and what
// limits it is the trip through LDS, not HBM: coalesced 16-byte register loads
// (8 rows x 128 bytes per wave instruction; loads in MFMA-fragment order touch
// two to four times as many cache lines per instruction and stream far slower)
// fetch each 128-byte K slice of the 128 weight rows and of XR token rows (XR =
// 16, 32, 64 or 128: the block rounded up) kSmallAhead slices ahead, and a slice is
// stored into a two-slice LDS ring just before its one barrier.  Eight waves
// form two groups of four; in a group, wave w takes neurons 32w .. 32w + 31,
// and the two groups take alternate k-steps of every slice, so each MFMA chain
// is half as long; group 1 parks its partial sums in LDS after the loop and
// group 0 adds them (a fixed order).  Up to 16 tokens the MFMA is 16x16x32
// (16 neurons x 16 tokens), above that 32x32x16 on 32-token blocks (those
// past the batch are skipped).  ReLU(g), rounded to bf16, is then staged in LDS as
// [token][128] and each wave packs every 8th token: lane l holds columns 2l,
// 2l + 1, and ballots give the slots in ascending column order.  Same stored
// values and format as the large-batch kernels.
constexpr int kSmallT = 64;   // one token block up to here
constexpr int kMidT = 2048;   // blocks of 128 tokens at most up to here

// Blocks of 128 tokens while all workgroups run in one generation (d_ff/128
// tiles x token blocks <= CUs: up to 512 tokens at d_ff = 8192, 1024 at
// 4096, 256 at 11008 on 256 CUs); a second generation made them slower than
// the 256-row tiles (1024 tokens at d_ff = 8192).
static bool use_small(const PackArgs& a) {
  if (a.T <= kSmallT) return true;
  if (a.T > kMidT) return false;
  int cus = lockstep_resident();
  if (cus <= 0) cus = 256;
  return static_cast<int64_t>(a.F / 128) * ((a.T + 127) / 128) <= cus;
}
constexpr int kSmallWaves = 8;   // two groups of 4 waves
constexpr int kSmallAhead = 4;   // K slices in flight in registers (d / 64 is a multiple of 8)

template <int XR>
__global__ __launch_bounds__(kSmallWaves * 64, 1) void gate_pack_small_kernel(PackArgs p) {
  constexpr bool kM16 = XR == 16;
  constexpr int kSlice = (128 + XR) * 128;  // one LDS slice: 128 weight rows, then XR token rows
  // load round q of wave w covers slice rows 8 (8q + w) + lane / 8; the last
  // round reaches past the slice for the higher waves ("short" waves): their
  // load there re-reads the clamped last row and is not stored, so every wave
  // issues the same number of loads and the compiler's wait counts stay exact
  constexpr int kRounds = (128 + XR + 8 * kSmallWaves - 1) / (8 * kSmallWaves);
  constexpr int kRoundsShort = (128 + XR) / (8 * kSmallWaves);
  extern __shared__ __align__(16) char lds[];
  __shared__ uint32_t ovf_s, nnz_s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31;
  constexpr int kNB = XR > 16 ? XR / 32 : 1;  // 32-token blocks (32x32x16 MFMAs)
  const int ng = wave & 3, kg = wave >> 2;  // neuron group (32 neurons), k-step group
  const int b = blockIdx.x;                 // TwELL tile
  const int n_t = p.F / 128;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * XR;                  // first token of the block
  const int T = static_cast<int>(min(static_cast<int64_t>(XR), p.T - t0));  // tokens in the block
  if (threadIdx.x == 0) {
    ovf_s = 0;
    nnz_s = 0;
  }
  const char* src[kRounds];
  int dst[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int r = min(8 * (kSmallWaves * q + wave) + (lane >> 3), 127 + XR);
    const char* base = r < 128 ? static_cast<const char*>(p.w_gate_t) +
                                     (static_cast<int64_t>(b) * 128 + r) * p.d * 2
                               : static_cast<const char*>(p.x) + (t0 + min(r - 128, T - 1)) * p.d * 2;
    src[q] = base + ((lane & 7) ^ lds_swz(r)) * 16;  // chunk c of the row lands in swizzled place
    dst[q] = r * 128 + (lane & 7) * 16;
  }
  const bool short_wave = 8 * (kSmallWaves * kRoundsShort + wave) >= 128 + XR;  // wave-uniform
  u32x4_t rg[kSmallAhead][kRounds];
  const int nk = p.d / 64;  // 128-byte slices
#pragma unroll
  for (int j = 0; j < kSmallAhead; ++j)
#pragma unroll
    for (int q = 0; q < kRounds; ++q) rg[j][q] = *reinterpret_cast<const u32x4_t*>(src[q] + j * 128);
  const int nb_live = (T + 31) / 32;  // token blocks holding tokens of the batch
  f32x16_t acc[kNB];  // 32x32x16: this wave's 32 neurons x tokens 32 tb .. 32 tb + 31
  f32x4_t a16[2];     // 16x16x32: neurons 32 ng + 16 h .. + 15 x 16 tokens
#pragma unroll
  for (int tb = 0; tb < kNB; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tb][r] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) a16[0][i] = a16[1][i] = 0.f;
  auto slice = [&](int kt, u32x4_t(&v)[kRounds], bool more) {
    // ring slot kt & 1 was last read in iteration kt - 2, which every wave
    // finished before the barrier of iteration kt - 1
    char* st = lds + (kt & 1) * kSlice;
#pragma unroll
    for (int q = 0; q < kRounds; ++q)
      if (q < kRoundsShort || !short_wave) *reinterpret_cast<u32x4_t*>(st + dst[q]) = v[q];
    if (more) {
#pragma unroll
      for (int q = 0; q < kRounds; ++q)
        v[q] = *reinterpret_cast<const u32x4_t*>(src[q] + static_cast<int64_t>(kt + kSmallAhead) * 128);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kM16) {
      // k32 step kg of the slice: lane l supplies 8 k-values (chunk 4 kg + l / 16) of
      // its neuron (A) and its token (B) row l % 16
      const int c = 4 * kg + (lane >> 4);
      const u32x4_t fb = *reinterpret_cast<const u32x4_t*>(st + lds_off(128 + (lane & 15), c));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t fa = *reinterpret_cast<const u32x4_t*>(st + lds_off(32 * ng + 16 * h + (lane & 15), c));
        a16[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa),
                                                        __builtin_bit_cast(bf16x8_t, fb), a16[h], 0, 0, 0);
      }
    } else {
      // k16 steps kg and kg + 2 of the slice; tokens past XR (past T) read the
      // last loaded token row, their outputs are discarded
      Frag<EBf16> fa[2], fb[2][kNB];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        read_frag256(fa[j], st, 32 * ng + li, kg + 2 * j, lane);
#pragma unroll
        for (int tb = 0; tb < kNB; ++tb)
          if (tb < nb_live) read_frag256(fb[j][tb], st, 128 + min(32 * tb + li, XR - 1), kg + 2 * j, lane);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int tb = 0; tb < kNB; ++tb)
          if (tb < nb_live) mfma_k16(acc[tb], fa[j], fb[j][tb]);
    }
  };
  // the last kSmallAhead slices issue no loads (peeled, so the loop's loads are unconditional)
  for (int kt0 = 0; kt0 < nk - kSmallAhead; kt0 += kSmallAhead) {
#pragma unroll
    for (int j = 0; j < kSmallAhead; ++j) slice(kt0 + j, rg[j], true);
  }
#pragma unroll
  for (int j = 0; j < kSmallAhead; ++j) slice(nk - kSmallAhead + j, rg[j], false);
  __syncthreads();  // every wave past its last ring reads: reuse the LDS
  // group 1's partials at [token block][wave ng][register][lane] (16 KB per
  // token block), then the staged rows [XR][128] bf16
  float* red = reinterpret_cast<float*>(lds);
  uint16_t(*gl)[128] = reinterpret_cast<uint16_t(*)[128]>(lds + kNB * 16 * 1024);
  if (kg == 1) {
    float* o = red + ng * 1024 + lane;
    if constexpr (kM16) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[(4 * h + i) * 64] = a16[h][i];
    } else {
#pragma unroll
      for (int tb = 0; tb < kNB; ++tb)
        if (tb < nb_live) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[tb * 4096 + r * 64] = acc[tb][r];
        }
    }
  }
  __syncthreads();
  if (kg == 0) {
    const float* o = red + ng * 1024 + lane;
    if constexpr (kM16) {
      // 16x16 accumulator: register i of lane l holds row 4 (l / 16) + i, column l % 16
      const int tok = lane & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = a16[h][i] + o[(4 * h + i) * 64];
          if (tok < T)
            gl[tok][32 * ng + 16 * h + 4 * (lane >> 4) + i] =
                static_cast<uint16_t>(round_store<EBf16>(g > 0.f ? g : 0.f).bits);
        }
    } else {
      // acc register r of lane l: neuron 32 ng + acc_row(r, l), token 32 tb + l % 32
#pragma unroll
      for (int tb = 0; tb < kNB; ++tb)
        if (tb < nb_live) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float g = acc[tb][r] + o[tb * 4096 + r * 64];
            if (32 * tb + li < T)
              gl[32 * tb + li][32 * ng + acc_row(r, lane)] =
                  static_cast<uint16_t>(round_store<EBf16>(g > 0.f ? g : 0.f).bits);
          }
        }
    }
  }
  __syncthreads();
  // pack: wave w takes tokens w, w + 8, ...; lane l holds columns 2l and 2l + 1
  const int C = p.C;
  uint32_t ovf = 0, nnz = 0;
  for (int t = wave; t < T; t += kSmallWaves) {
    const uint32_t v0 = gl[t][2 * lane], v1 = gl[t][2 * lane + 1];
    if (p.gate_dbg) {
      uint16_t* gd = static_cast<uint16_t*>(p.gate_dbg) + (t0 + t) * p.F + b * 128 + 2 * lane;
      gd[0] = static_cast<uint16_t>(v0);
      gd[1] = static_cast<uint16_t>(v1);
    }
    const int nz0 = v0 != 0u, nz1 = v1 != 0u;
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(nz0 + nz1 >= 1);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(nz0 + nz1 >= 2);
    const int excl = static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m1 >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m1), 0u))) +
                     static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m2 >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m2), 0u)));
    const int count = static_cast<int>(__popcll(m1) + __popcll(m2));
    const int64_t unit = (t0 + t) * n_t + b;
    const int64_t rec = unit * C;
    if (lane == 0) p.count[unit] = count;
    if (nz0 && excl < C) {
      p.idx[rec + excl] = static_cast<uint8_t>(2 * lane);
      static_cast<uint16_t*>(p.val)[rec + excl] = static_cast<uint16_t>(v0);
    }
    if (nz1 && excl + nz0 < C) {
      p.idx[rec + excl + nz0] = static_cast<uint8_t>(2 * lane + 1);
      static_cast<uint16_t*>(p.val)[rec + excl + nz0] = static_cast<uint16_t>(v1);
    }
    for (int sl = lane; sl < C; sl += 64)  // slots past the stored entries: (0, +0)
      if (sl >= count) {
        p.idx[rec + sl] = 0;
        static_cast<uint16_t*>(p.val)[rec + sl] = 0;
      }
    ovf += count > C ? 1u : 0u;
    nnz += static_cast<uint32_t>(count);
  }
  if (p.stats) {
    if (lane == 0) {
      atomicAdd(&ovf_s, ovf);
      atomicAdd(&nnz_s, nnz);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      if (ovf_s) atomicAdd(p.stats + 0, static_cast<unsigned long long>(ovf_s));
      if (nnz_s) atomicAdd(p.stats + 1, static_cast<unsigned long long>(nnz_s));
    }
  }
}

template <int XR>
static hipError_t launch_pack_small_t(const PackArgs& a, hipStream_t s) {
  constexpr int kRing = 2 * (128 + XR) * 128;
  constexpr int kNB = XR > 16 ? XR / 32 : 1;
  constexpr int kEpilogue = kNB * 16 * 1024 + (XR < 64 ? 64 : XR) * 128 * 2;  // partial sums, then staged rows
  constexpr int lds = kRing > kEpilogue ? kRing : kEpilogue;
  static_assert(lds + 64 <= 160 * 1024, "LDS of one workgroup");
  static_assert(kSmallWaves == 8 && 8 % kSmallAhead == 0, "two wave groups; slices a multiple of the prefetch");
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_pack_small_kernel<XR>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const unsigned blocks = static_cast<unsigned>((a.T + XR - 1) / XR);
  hipLaunchKernelGGL((gate_pack_small_kernel<XR>), dim3(a.F / 128, blocks), dim3(kSmallWaves * 64), lds, s, a);
  return hipGetLastError();
}

static hipError_t launch_pack_small(const PackArgs& a, hipStream_t s) {
  if (a.T <= 16) return launch_pack_small_t<16>(a, s);
  if (a.T <= 32) return launch_pack_small_t<32>(a, s);
  if (a.T <= kSmallT) return launch_pack_small_t<64>(a, s);
  return launch_pack_small_t<128>(a, s);
}

template <class E>
static hipError_t launch_pack_e(const PackArgs& a, hipStream_t s) {
  if (E::kBytes == 2 && a.tile_n == 128 && use_small(a)) return launch_pack_small(a, s);
  const bool dbg = a.gate_dbg != nullptr;
  if (a.tile_n == 128) return dbg ? launch_pack256_t<E, true>(a, s) : launch_pack256_t<E, false>(a, s);
  return dbg ? launch_pack64_t<E, true>(a, s) : launch_pack64_t<E, false>(a, s);
}

hipError_t launch_gate_pack(const PackArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_pack_e<EBf16>(a, s) : launch_pack_e<EF32>(a, s);
}

}  // namespace twell
