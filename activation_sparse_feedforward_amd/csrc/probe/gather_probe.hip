// Gather-ceiling probe for the fused up/down kernel's access pattern.
//
// The fused kernel (TwELL page "Sakana AI and NVIDIA introduce TwELL with
// CUDA kernels...", section "¿Qué hace distinto a TwELL frente a ELL
// clásico?": one fused kernel gathers the weight rows of the active neurons)
// spends its time fetching whole weight rows: per active (token, neuron) pair
// one row of W_up^T and one of W_down, 2 * d_model bytes each at bf16.  This
// probe moves the same rows the same way -- one workgroup per CU of 16 waves
// (8 for rows wider than 4 KB, as the fused kernel), every lane loading
// 16-byte pieces of the row, two rows per step -- without any arithmetic, so
// its rate is what the memory system gives that pattern:
//   mode 0 (random): each wave picks its rows at random from both matrices,
//          so nearly every row comes from past L2 (the MALL holds both);
//   mode 1 (XCD-shared): the waves of one XCD (workgroup id mod 8, the
//          dispatcher's round-robin) read the same row sequence at about the
//          same time, so most rows are served by that XCD's L2.
// Measurement only: the library never calls it.  Each wave folds what it
// loaded into one word written to out[wave], so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ uint32_t mix(uint32_t v) {  // a 32-bit integer hash (murmur3 finaliser)
  v ^= v >> 16;
  v *= 0x85ebca6bu;
  v ^= v >> 13;
  v *= 0xc2b2ae35u;
  v ^= v >> 16;
  return v;
}

// NV 16-byte pieces per lane per row (row = NV * 64 * 16 bytes); U steps of two
// rows in flight per wave; kWaves waves per workgroup.
template <int NV, int U, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void gather_probe_kernel(const char* a, const char* b, int64_t rows,
                                                                   int steps, int shared, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t gw = blockIdx.x * kWaves + wave;
  const uint32_t seq = shared ? (blockIdx.x & 7u) : gw;  // whose row sequence this wave follows
  constexpr int64_t kRowBytes = NV * 64 * 16;
  uint32_t acc = 0;
  for (int s = 0; s < steps; s += U) {
    u32x4 ra[U][NV], rb[U][NV];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const uint32_t h = mix(seq * 0x9e3779b9u + static_cast<uint32_t>(s + q) * 0x7f4a7c15u + 1u);
      const int64_t r = static_cast<int64_t>(h % static_cast<uint32_t>(rows));
      const u32x4* pa = reinterpret_cast<const u32x4*>(a + r * kRowBytes);
      const u32x4* pb = reinterpret_cast<const u32x4*>(b + r * kRowBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        ra[q][v] = pa[v * 64 + lane];
        rb[q][v] = pb[v * 64 + lane];
      }
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4 t = ra[q][v] ^ rb[q][v];
        acc ^= t.x ^ t.y ^ t.z ^ t.w;
      }
  }
  acc ^= __shfl_xor(acc, 32);
  if (lane == 0) out[gw] = acc;
}

// 96 KB of (unused) LDS per workgroup keeps one workgroup per CU, as in the
// fused kernel.
constexpr int kPinLds = 96 * 1024;

template <int NV, int U, int kWaves>
int launch_u(const char* a, const char* b, int64_t rows, int steps, int shared, int blocks, uint32_t* out,
             hipStream_t s) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gather_probe_kernel<NV, U, kWaves>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kPinLds) != hipSuccess)
    return 3;
  hipLaunchKernelGGL((gather_probe_kernel<NV, U, kWaves>), dim3(blocks), dim3(kWaves * 64), kPinLds, s, a, b, rows,
                     steps, shared, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// the deeper case keeps eight rows in flight per wave up to 4 KB rows and four
// above (whose 8-wave workgroups have twice the registers per wave)
template <int NV>
int launch_nv(const char* a, const char* b, int64_t rows, int steps, int shared, int in_flight, int blocks,
              uint32_t* out, hipStream_t s) {
  if constexpr (NV <= 4)
    return in_flight >= 4 ? launch_u<NV, 4, 16>(a, b, rows, steps, shared, blocks, out, s)
                          : launch_u<NV, 1, 16>(a, b, rows, steps, shared, blocks, out, s);
  else
    return in_flight >= 4 ? launch_u<NV, 2, 8>(a, b, rows, steps, shared, blocks, out, s)
                          : launch_u<NV, 1, 8>(a, b, rows, steps, shared, blocks, out, s);
}

}  // namespace

// a, b: two row-major matrices of `rows` rows of row_bytes (1024, 2048, 4096,
// 5120, 6144, 7168 or 8192) each; out: blocks * 16 words.  steps: multiple of
// 4.  in_flight: 1 (two rows per wave in flight, as the fused kernel) or 4
// (eight rows; four for rows wider than 4 KB).  Returns 0 on success, non-zero
// for a bad argument or a failed launch.
extern "C" int twell_probe_gather(const void* a, const void* b, int64_t rows, int row_bytes, int steps, int shared,
                                  int in_flight, int blocks, uint32_t* out, void* stream) {
  if (!a || !b || !out || rows <= 0 || rows > (int64_t(1) << 31) || steps <= 0 || steps % 4 || blocks <= 0)
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  switch (row_bytes) {
    case 1024: return launch_nv<1>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 2048: return launch_nv<2>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 4096: return launch_nv<4>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 5120: return launch_nv<5>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 6144: return launch_nv<6>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 7168: return launch_nv<7>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
    case 8192: return launch_nv<8>(pa, pb, rows, steps, shared, in_flight, blocks, out, s);
  }
  return 2;
}
