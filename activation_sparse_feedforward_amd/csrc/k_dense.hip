// Dense MFMA FFN kernels: the library's own dense baseline and the dense
// fallback of the hybrid format.
//
// The TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA kernels...")
// measures its sparse path against the dense Tensor-Core FFN (section "¿Cuál
// es el problema que TwELL resuelve?") and, for training, routes rows with too
// many non-zeros to a dense fallback (section "¿Qué hace distinto a TwELL
// frente a ELL clásico?").  Both use these two kernels:
//   gateup: one GEMM whose 64-wide B tile is 32 gate rows + the same 32 up
//           rows, so a lane holds g and u of the same (row, neuron) in
//           matching accumulator registers; epilogue h = ReLU(g) * u;
//   down:   y = h . W_down with W_down read [d_ff x d_model] (N contiguous)
//           and transposed into the K-contiguous LDS layout on the way in.
// Both take an optional row table (gather x / scatter y) and an optional
// device-side row count, so the fallback can run on rows chosen on the GPU
// without a host round trip: workgroups past the count exit at once.
//
// The full dense FFN runs the same two steps on the 256 x 256 core of
// gemm256.hpp instead (gateup256, down256); its down GEMM reads W_down^T,
// which transpose_kernel writes into the caller's workspace first (the core
// wants both operands K-contiguous).
#include "gemm256.hpp"
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

template <class E>
__global__ __launch_bounds__(kThreads, 2) void gateup_kernel(GateUpArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.M;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n_rows) return;
  // 32 neurons per workgroup: the fallback rows are few (one 256-row block at
  // the training workload), so d_ff / 32 workgroups are what fills the chip
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 32;

  KRowLoader<E, kBM> la;
  la.init(p.x, p.d, m0, n_rows, p.rows);
  struct {
    KRowLoader<E, 32> g, u;
    __device__ void load(int kt) { g.load(kt); u.load(kt); }
    __device__ void store(char* l, int) const { g.store(l, 0); u.store(l, 32); }
  } lb;
  lb.g.init(p.w_gate_t, p.d, j0, p.F, nullptr);
  lb.u.init(p.w_up_t, p.d, j0, p.F, nullptr);
  Acc<64> acc;
  gemm_mainloop<E, 64>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);

  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
      const float g = acc.c[mb][0][r];
      const float h = (g > 0.f ? g : 0.f) * acc.c[mb][1][r];
      store_bits<E>(p.h, m * p.F + j0 + (lane & 31), round_store<E>(h).bits);
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
  // split-K: blockIdx.z takes K rows [k0, k0 + ks) of h's columns / W_down's rows
  const int splits = p.splits > 1 ? p.splits : 1;
  const int64_t ks = p.F / splits, k0 = static_cast<int64_t>(blockIdx.z) * ks;

  KRowLoader<E, kBM> la;
  la.init(static_cast<const char*>(p.h) + k0 * E::kBytes, p.F, m0, n_rows, nullptr);
  MNColLoader<E, 128> lb;
  lb.init(static_cast<const char*>(p.w_down) + k0 * p.d * E::kBytes, p.d, n0, p.d, ks);
  Acc<128> acc;
  gemm_mainloop<E, 128>(la, lb, static_cast<int>(ks / KRowLoader<E, kBM>::kSliceElems), lds, acc);

  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
      if (splits > 1) {
        float* o = p.part + (static_cast<int64_t>(blockIdx.z) * p.M + m) * p.d + n0 + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[nb * 32] = acc.c[mb][nb][r];
        continue;
      }
      const int64_t row = p.rows ? static_cast<int64_t>(p.rows[m]) : m;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        store_bits<E>(p.y, row * p.d + n0 + nb * 32 + (lane & 31), round_store<E>(acc.c[mb][nb][r]).bits);
    }
  }
}

// Fixed-order sum of split-K partials, rounded and scattered to the output
// rows; 4 consecutive columns per thread.  Threads past n_rows exit.
template <class E>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits, int64_t M,
                                                            const int32_t* n_rows_dev, const int32_t* rows,
                                                            void* out, int d) {
  const int64_t n_rows = n_rows_dev ? static_cast<int64_t>(*n_rows_dev) : M;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t m = i / d;
  if (m >= n_rows || m >= M) return;
  const int64_t n = i - m * d;
  float4 acc = *reinterpret_cast<const float4*>(part + m * d + n);
  for (int s = 1; s < splits; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + (static_cast<int64_t>(s) * M + m) * d + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const int64_t o = (rows ? static_cast<int64_t>(rows[m]) : m) * d + n;
  store_bits<E>(out, o + 0, round_store<E>(acc.x).bits);
  store_bits<E>(out, o + 1, round_store<E>(acc.y).bits);
  store_bits<E>(out, o + 2, round_store<E>(acc.z).bits);
  store_bits<E>(out, o + 3, round_store<E>(acc.w).bits);
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, const int32_t* n_rows_dev,
                                const int32_t* rows, void* out, int d, int dtype, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((M * d / 4 + 255) / 256);
  if (blocks == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((splitk_reduce_kernel<EBf16>), dim3(blocks), dim3(256), 0, s, part, splits, M, n_rows_dev,
                       rows, out, d);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<EF32>), dim3(blocks), dim3(256), 0, s, part, splits, M, n_rows_dev,
                       rows, out, d);
  return hipGetLastError();
}

// gate|up on the 256 x 256 core: workgroup tile = 256 rows x 128 neurons.  The
// B tile interleaves 64 gate rows and the same 64 up rows per wave column
// (DirectRows::init_split), so g and u of one (row, neuron) sit in
// accumulator blocks j and j + 2 of the same lane.  1-D grid of
// n_mt * ceil(F/128); with F an odd multiple of 64 the last tile's upper half
// is clamped on load and not stored.
template <class E>
__global__ __launch_bounds__(256, 1) void gateup256_kernel(GateUpArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.M;
  const int n_nt = (p.F + 127) / 128;
  const int n_mt = static_cast<int>(gridDim.x) / n_nt;
  int mt, nt;
  tile_coords_256(n_mt, n_nt, mt, nt);
  const int64_t m0 = static_cast<int64_t>(mt) * kT256;
  if (m0 >= n_rows) return;
  const int64_t n0 = static_cast<int64_t>(nt) * 128;
  DirectRows<E> la, lb;
  la.init(p.x, p.d, m0, n_rows, p.rows);
  lb.init_split(p.w_gate_t, p.w_up_t, p.d, n0, p.F);
  Acc256 acc;
  gemm256_mainloop<E>(la, lb, p.d / (128 / E::kBytes), lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wrow0 = m0 + (wave >> 1) * 128;
  const int64_t col0 = n0 + (wave & 1) * 64 + (lane & 31);
  if (n0 + (wave & 1) * 64 >= p.F) return;  // no barrier follows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + i * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float g = acc.c[i][j][r];
        const float h = (g > 0.f ? g : 0.f) * acc.c[i][j + 2][r];
        store_bits<E>(p.h, m * p.F + col0 + j * 32, round_store<E>(h).bits);
      }
    }
  }
}

// y[row(m), :] = h[m, :] . W_down on the 256 x 256 core, with W_down^T
// ([d_model x d_ff], K-contiguous) in p.w_down_t.  1-D grid of n_mt * d/256.
template <class E>
__global__ __launch_bounds__(256, 1) void down256_kernel(DownArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.M;
  const int n_nt = p.d / kT256;
  const int n_mt = static_cast<int>(gridDim.x) / n_nt;
  int mt, nt;
  tile_coords_256(n_mt, n_nt, mt, nt);
  const int64_t m0 = static_cast<int64_t>(mt) * kT256;
  if (m0 >= n_rows) return;
  const int64_t n0 = static_cast<int64_t>(nt) * kT256;
  DirectRows<E> la, lb;
  la.init(p.h, p.F, m0, n_rows, nullptr);
  lb.init(p.w_down_t, p.F, n0, p.d, nullptr);
  Acc256 acc;
  gemm256_mainloop<E>(la, lb, p.F / (128 / E::kBytes), lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wrow0 = m0 + (wave >> 1) * 128;
  const int64_t col0 = n0 + (wave & 1) * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + i * 32 + acc_row(r, lane);
      if (m >= n_rows) continue;
      const int64_t row = p.rows ? static_cast<int64_t>(p.rows[m]) : m;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_bits<E>(p.y, row * p.d + col0 + j * 32, round_store<E>(acc.c[i][j][r]).bits);
    }
  }
}

// dst[c][r] = src[r][c] for a [rows x cols] matrix; 64 x 64 tiles through LDS.
// rows and cols are multiples of 64; grid (cols/64, rows/64), 256 threads.
template <class E>
__global__ __launch_bounds__(256) void transpose_kernel(const void* src, void* dst, int rows, int cols) {
  __shared__ uint32_t tile[64][65];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t o = (r0 + i) * cols + c0 + tx;
    tile[i][tx] = E::kBytes == 2 ? static_cast<const uint16_t*>(src)[o] : static_cast<const uint32_t*>(src)[o];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) store_bits<E>(dst, (c0 + i) * rows + r0 + tx, tile[tx][i]);
}

template <class E>
static hipError_t launch_dense256_t(const GateUpArgs& g, const DownArgs& dn, hipStream_t s) {
  static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&gateup256_kernel<E>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, kLds256);
  static const hipError_t a2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&down256_kernel<E>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, kLds256);
  if (a1 != hipSuccess) return a1;
  if (a2 != hipSuccess) return a2;
  const unsigned n_mt = static_cast<unsigned>((g.M + kT256 - 1) / kT256);
  hipLaunchKernelGGL((transpose_kernel<E>), dim3(dn.d / 64, dn.F / 64), dim3(256), 0, s, dn.w_down,
                     const_cast<void*>(dn.w_down_t), dn.F, dn.d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gateup256_kernel<E>), dim3(n_mt * ((g.F + 127) / 128)), dim3(256), kLds256, s, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((down256_kernel<E>), dim3(n_mt * (dn.d / kT256)), dim3(256), kLds256, s, dn);
  return hipGetLastError();
}

hipError_t launch_dense256(const GateUpArgs& g, const DownArgs& dn, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_dense256_t<EBf16>(g, dn, s) : launch_dense256_t<EF32>(g, dn, s);
}

template <class E>
static hipError_t launch_gateup_t(const GateUpArgs& a, hipStream_t s) {
  dim3 grid(a.F / 32, static_cast<unsigned>((a.M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gateup_kernel<E>), grid, dim3(kThreads), (kBM + 64) * 128, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_down_t(const DownArgs& a, hipStream_t s) {
  const int splits = a.splits > 1 ? a.splits : 1;
  dim3 grid(a.d / 128, static_cast<unsigned>((a.M + kBM - 1) / kBM), splits);
  hipLaunchKernelGGL((down_kernel<E>), grid, dim3(kThreads), (kBM + 128) * 128, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(a.part, splits, a.M, a.n_rows_dev, a.rows, a.y, a.d, E::kBytes == 2 ? 1 : 0, s);
}

hipError_t launch_gateup(const GateUpArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_gateup_t<EBf16>(a, s) : launch_gateup_t<EF32>(a, s);
}
hipError_t launch_down(const DownArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_down_t<EBf16>(a, s) : launch_down_t<EF32>(a, s);
}

}  // namespace twell
