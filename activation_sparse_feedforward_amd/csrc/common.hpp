// Common device-side definitions for libtwell (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- element types
// Storage element traits.  Arithmetic is always fp32.
struct EBf16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};
struct EF32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes, returned as a wave-uniform value.  Butterflies inside
// each row of 16 lanes leave every lane with its row's sum; the gfx9 row
// broadcasts then carry row 0 into row 1 and row 2 into row 3 (row_bcast:15),
// and row 1 into rows 2 and 3 (row_bcast:31), so lane 63 holds the total: no
// LDS round trip (a cross-row shuffle goes through ds_bpermute).
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror: combine the two quads of each 8
  v = dpp_add<0x140>(v);  // row_mirror: combine the two 8-lane halves of each row of 16
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// v of the lane that DPP control CTRL names, 0 where that lane is outside
// the row (row shifts) or the row is masked off.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_take(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes; every lane must be active.  Shifts
// by 1, 2, 4 and 8 lanes inside each row of 16 build the row-local sums, then
// the row broadcasts add row 0's total into row 1 and row 2's into row 3, and
// rows 0-1's total into rows 2 and 3.  No LDS round trip.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_take<0x111>(v);       // row_shr:1
  v += dpp_take<0x112>(v);       // row_shr:2
  v += dpp_take<0x114>(v);       // row_shr:4
  v += dpp_take<0x118>(v);       // row_shr:8
  v += dpp_take<0x142, 0xa>(v);  // row_bcast:15
  v += dpp_take<0x143, 0xc>(v);  // row_bcast:31
  return v;
}

// Lane 63's value (an inclusive scan's total) as a wave-uniform value.
__device__ __forceinline__ int wave_last(int v) { return __builtin_amdgcn_readlane(v, 63); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// y += c * w over one 16-byte piece of a row held in storage form, y in fp32.
// bf16: c is rounded to bf16 once (the precision in which a dense bf16 path
// stores the hidden activations and their gradients before the next
// product) and every element is a packed-pair dot product of the row's bf16
// pair with (c, 0) or (0, c): the product of two bf16 values is exact in
// fp32, so each element still takes one fp32 rounding, and the row needs no
// unpacking.  fp32: plain FMAs.  (The 16-byte vector is bit-cast whole to
// bf16x8 before taking pairs: casting an element of the 32-bit vector
// directly was compiled to always read element 0.)
template <class E> struct AxpyCoef;
template <> struct AxpyCoef<EBf16> {
  bf16x2_t lo, hi;  // (c, 0) and (0, c)
  __device__ __forceinline__ explicit AxpyCoef(float c) {
    const uint32_t b = f32_to_bf16_bits(c);
    lo = __builtin_bit_cast(bf16x2_t, b);
    hi = __builtin_bit_cast(bf16x2_t, b << 16);
  }
  __device__ __forceinline__ void axpy(const u32x4_t& w, float* y) const {
    const bf16x8_t wh = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t pr{wh[2 * i], wh[2 * i + 1]};
      y[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(pr, lo, y[2 * i], false);
      y[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, hi, y[2 * i + 1], false);
    }
  }
};
template <> struct AxpyCoef<EF32> {
  float c;
  __device__ __forceinline__ explicit AxpyCoef(float v) : c(v) {}
  __device__ __forceinline__ void axpy(const u32x4_t& w, float* y) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = fmaf(c, __uint_as_float(w[i]), y[i]);
  }
};

template <class E> __device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<EBf16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<EF32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}

// Round an fp32 value to the storage dtype and return (stored bits as uint32, value as fp32).
template <class E> struct Rounded { uint32_t bits; float value; };
template <class E> __device__ __forceinline__ Rounded<E> round_store(float v);
template <> __device__ __forceinline__ Rounded<EBf16> round_store<EBf16>(float v) {
  uint32_t b = f32_to_bf16_bits(v);
  return {b, bf16_bits_to_f32(b)};
}
template <> __device__ __forceinline__ Rounded<EF32> round_store<EF32>(float v) {
  return {__float_as_uint(v), v};
}

template <class E> __device__ __forceinline__ void store_bits(void* p, int64_t i, uint32_t bits);
template <> __device__ __forceinline__ void store_bits<EBf16>(void* p, int64_t i, uint32_t bits) {
  static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(bits);
}
template <> __device__ __forceinline__ void store_bits<EF32>(void* p, int64_t i, uint32_t bits) {
  static_cast<uint32_t*>(p)[i] = bits;
}

// ---------------------------------------------------------------- MFMA 32x32 step
// One "k16 step" of a 32x32 output block: each lane supplies 8 consecutive K
// elements of its A row (lane % 32) and of its B column (lane % 32), the two
// 8-element groups of a lane covering k = 8*(lane/32) .. +7.  Because A and B
// use the same lane->k assignment, the sum over k is complete whatever order
// the hardware pairs them in.
//   bf16: one v_mfma_f32_32x32x16_bf16 (16 bytes / lane / operand)
//   fp32: eight v_mfma_f32_32x32x2_f32 (32 bytes / lane / operand)
template <class E> struct Frag;
template <> struct Frag<EBf16> { u32x4_t v; };
template <> struct Frag<EF32> { u32x4_t v[2]; };

__device__ __forceinline__ void mfma_k16(f32x16_t& acc, const Frag<EBf16>& a, const Frag<EBf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_k16(f32x16_t& acc, const Frag<EF32>& a, const Frag<EF32>& b) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.v[h][i]), __uint_as_float(b.v[h][i]),
                                                 acc, 0, 0, 0);
    }
  }
}

// Accumulator layout of a 32x32 block (16 fp32 per lane): register r of lane l
// holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------- LDS tile layout
// An operand tile in LDS is R rows x 128 bytes (the K extent of one main-loop
// step: 64 bf16 or 32 fp32), K contiguous within a row.  The eight 16-byte
// chunks of a row are XOR-permuted so that (a) eight consecutive rows read at
// the same chunk hit eight different bank groups (fragment reads) and (b)
// writes of one element column across rows 8 apart do too (transposing stores).
__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ lds_swz(row)) << 4); }

}  // namespace twell
