// Dense MFMA FFN kernels: the library's own dense baseline and the dense
// fallback of the hybrid format.
//
// The TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA kernels...")
// measures its sparse path against the dense Tensor-Core FFN (section "¿Cuál
// es el problema que TwELL resuelve?") and, for training, routes rows with too
// many non-zeros to a dense fallback (section "¿Qué hace distinto a TwELL
// frente a ELL clásico?").  Both use these two kernels:
//   gateup: one GEMM whose 128-wide B tile is 64 gate rows + the same 64 up
//           rows, so a lane holds g and u of the same (row, neuron) in
//           matching accumulator registers; epilogue h = ReLU(g) * u;
//   down:   y = h . W_down with W_down read [d_ff x d_model] (N contiguous)
//           and transposed into the K-contiguous LDS layout on the way in.
// Both take an optional row table (gather x / scatter y) and an optional
// device-side row count, so the fallback can run on rows chosen on the GPU
// without a host round trip: workgroups past the count exit at once.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

template <class E>
__global__ __launch_bounds__(kThreads, 2) void gateup_kernel(GateUpArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.M;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n_rows) return;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;

  KRowLoader<E, kBM> la;
  la.init(p.x, p.d, m0, n_rows, p.rows);
  struct {
    KRowLoader<E, 64> g, u;
    __device__ void load(int kt) { g.load(kt); u.load(kt); }
    __device__ void store(char* l, int) const { g.store(l, 0); u.store(l, 64); }
  } lb;
  lb.g.init(p.w_gate_t, p.d, j0, p.F, nullptr);
  lb.u.init(p.w_up_t, p.d, j0, p.F, nullptr);
  Acc<128> acc;
  gemm_mainloop<E, 128>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);

  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float g = acc.c[mb][nb][r];
        const float h = (g > 0.f ? g : 0.f) * acc.c[mb][nb + 2][r];
        store_bits<E>(p.h, m * p.F + j0 + nb * 32 + (lane & 31), round_store<E>(h).bits);
      }
    }
  }
}

template <class E>
__global__ __launch_bounds__(kThreads, 2) void down_kernel(DownArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.M;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n_rows) return;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128;

  KRowLoader<E, kBM> la;
  la.init(p.h, p.F, m0, n_rows, nullptr);
  MNColLoader<E, 128> lb;
  lb.init(p.w_down, p.d, n0, p.d, p.F);
  Acc<128> acc;
  gemm_mainloop<E, 128>(la, lb, p.F / KRowLoader<E, kBM>::kSliceElems, lds, acc);

  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
      const int64_t row = p.rows ? static_cast<int64_t>(p.rows[m]) : m;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        store_bits<E>(p.y, row * p.d + n0 + nb * 32 + (lane & 31), round_store<E>(acc.c[mb][nb][r]).bits);
    }
  }
}

template <class E>
static hipError_t launch_gateup_t(const GateUpArgs& a, hipStream_t s) {
  dim3 grid(a.F / 64, static_cast<unsigned>((a.M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gateup_kernel<E>), grid, dim3(kThreads), (kBM + 128) * 128, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_down_t(const DownArgs& a, hipStream_t s) {
  dim3 grid(a.d / 128, static_cast<unsigned>((a.M + kBM - 1) / kBM));
  hipLaunchKernelGGL((down_kernel<E>), grid, dim3(kThreads), (kBM + 128) * 128, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup(const GateUpArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_gateup_t<EBf16>(a, s) : launch_gateup_t<EF32>(a, s);
}
hipError_t launch_down(const DownArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_down_t<EBf16>(a, s) : launch_down_t<EF32>(a, s);
}

}  // namespace twell
