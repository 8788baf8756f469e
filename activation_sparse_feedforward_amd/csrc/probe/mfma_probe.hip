// MFMA-ceiling probe for the gate kernel's matrix-core work.
//
// The gate GEMM (TwELL page "Sakana AI and NVIDIA introduce TwELL with CUDA
// kernels...", section "¿Qué hace distinto a TwELL frente a ELL clásico?":
// the existing matmul kernel, with the sparse format written by its
// epilogue) issues v_mfma_f32_32x32x16_bf16 from one wave per SIMD, one
// workgroup of four waves per CU, each wave cycling through 16 independent
// 32x32 accumulator blocks held in AGPRs.  This probe runs only that: the same
// occupancy and the same instruction on the same 16 accumulators, with
// operands held in registers (never touching memory during the loop), so its
// rate is what the matrix cores deliver under a full, sustained MFMA load --
// the practical ceiling the gate kernel's main loop can approach.  Operands
// are either one constant fragment pair (few bits toggle: the issue-rate
// ceiling) or eight A and eight B fragments of random bits read once from
// `frags` and cycled through (the switching of a real GEMM, and the clock
// the chip can hold with it).  Each wave also reads the
// shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around its loop, so the clock the chip held during the run
// can be computed.  Measurement only: the library never calls it.  Each wave
// folds its accumulators into one word written to out[wave], so no MFMA can
// be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlocks = 16;  // accumulator blocks per wave, as the gate kernel's 4 x 4

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kRandom>
__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(int iters, const u32x4* frags, uint32_t* out,
                                                            uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  constexpr int kF = kRandom ? 8 : 1;  // fragment pairs cycled through
  bf16x8 a[kF], b[kF];
  if constexpr (kRandom) {
#pragma unroll
    for (int f = 0; f < kF; ++f) {  // frags: [16][64] 16-byte pieces (eight A, then eight B)
      a[f] = __builtin_bit_cast(bf16x8, frags[f * 64 + lane]);
      b[f] = __builtin_bit_cast(bf16x8, frags[(8 + f) * 64 + lane]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // small, lane-dependent operands: the sums stay far from overflow
      a[0][i] = static_cast<__bf16>(static_cast<float>((lane + i) & 7) * 0.0009765625f);
      b[0][i] = static_cast<__bf16>(static_cast<float>((lane * 3 + i) & 7) * 0.0009765625f);
    }
  }
  f32x16 acc[kBlocks];
#pragma unroll
  for (int m = 0; m < kBlocks; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
    // like the gate kernel's k-steps: block m takes A fragment m / 4 and B fragment m % 4, and
    // consecutive k-steps use other fragments (with random operands: fragments 0-3, then 4-7)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < kBlocks; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[((m >> 2) + 4 * h) % kF], b[((m & 3) + 4 * h) % kF], acc[m],
                                                         0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < kBlocks; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[m][r];
  out[gw * 64 + lane] = __float_as_uint(s);
  if (lane == 0) {
    clocks[gw * 2 + 0] = t1 - t0;  // shader-clock cycles of the loop
    clocks[gw * 2 + 1] = r1 - r0;  // 100 MHz ticks of the loop
  }
}

}  // namespace

// blocks workgroups of 4 waves (one per CU for the gate kernel's occupancy),
// each wave running iters (even) x 16 MFMAs of 32 x 32 x 16 (32,768 FLOP each).
// frags: NULL for constant operands, else 16 KB of operand bits (16 x 64
// pieces of 16 bytes; every piece should hold finite bf16 values).  out:
// blocks * 256 words; clocks: blocks * 8 64-bit words (per wave: shader
// cycles, then 100 MHz ticks).  Returns 0 on success, non-zero for a bad
// argument or a failed launch.
extern "C" int twell_probe_mfma(int iters, int blocks, const void* frags, uint32_t* out, uint64_t* clocks,
                                void* stream) {
  if (iters <= 0 || iters % 2 || blocks <= 0 || !out || !clocks) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* f = static_cast<const u32x4*>(frags);
  if (f)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, iters, f, out,
                       clocks);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, iters, f, out,
                       clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
