// Backward of the rows the hybrid format sent to the dense fallback, on MFMA.
//
// Same loss as the sparse backward (sum(y*dy) + l1 sum|h|, h = ReLU(g)*u); for
// these few rows everything is dense, so it is four GEMM launches over the
// gathered rows (n_dense is read on the device; workgroups past it exit):
//   gu:  g, u = x_d W_gate, x_d W_up (recomputed, fp32 into the workspace)
//   dh:  dh = dy_d W_down^T, epilogue: + l1 sign(h); du = dh a; dg = dh u [g>0]
//        -> dG, dU, H (dtype) in the workspace
//   dx:  dx_d = dG W_gate^T... in the stored layout: dx[t,k] = sum_j dG[m,j] W_gate^T[j,k]
//        + dU[m,j] W_up^T[j,k]; two K passes into one accumulator, rows scattered
//   dw:  dW_gate^T += dG^T x_d, dW_up^T += dU^T x_d, dW_down += H^T dy_d
//        (both operands MN-contiguous, K = n_dense, fp32 read-modify-write on
//        top of the sparse rows' contribution written before)
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

namespace {
__device__ __forceinline__ int64_t n_dense_of(const BwdArgs& p) { return static_cast<int64_t>(p.n_rows[1]); }
}  // namespace

template <class E>
__global__ __launch_bounds__(kThreads, 2) void bwd_gu_kernel(BwdArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n = n_dense_of(p);
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n) return;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
  KRowLoader<E, kBM> la;
  la.init(p.x, p.d, m0, n, p.dense_rows);
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
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int64_t o = m * p.F + j0 + nb * 32 + (lane & 31);
        p.g_d[o] = acc.c[mb][nb][r];
        p.u_d[o] = acc.c[mb][nb + 2][r];
      }
    }
}

template <class E>
__global__ __launch_bounds__(kThreads, 2) void bwd_dh_kernel(BwdArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n = n_dense_of(p);
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n) return;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 128;
  KRowLoader<E, kBM> la;
  la.init(p.dy, p.d, m0, n, p.dense_rows);
  KRowLoader<E, 128> lb;
  lb.init(p.w_down, p.d, j0, p.F, nullptr);
  Acc<128> acc;
  gemm_mainloop<E, 128>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);
  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int64_t j = j0 + nb * 32 + (lane & 31);
        if (j >= p.F) continue;  // d_ff need only be a multiple of 64
        const int64_t o = m * p.F + j;
        const float g = p.g_d[o], u = p.u_d[o];
        const float a = g > 0.f ? g : 0.f;
        const float h = a * u;
        const float sg = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
        const float dh = acc.c[mb][nb][r] + p.l1 * sg;
        store_bits<E>(p.du_d, o, round_store<E>(dh * a).bits);
        store_bits<E>(p.dg_d, o, round_store<E>(g > 0.f ? dh * u : 0.f).bits);
        store_bits<E>(p.h_d, o, round_store<E>(h).bits);
      }
    }
}

template <class E>
__global__ __launch_bounds__(kThreads, 2) void bwd_dx_kernel(BwdArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n = n_dense_of(p);
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n) return;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128;
  // split-K over the neurons: blockIdx.z takes j in [k0, k0 + ks)
  const int splits = p.dx_splits > 1 ? p.dx_splits : 1;
  const int64_t ks = p.F / splits, k0 = static_cast<int64_t>(blockIdx.z) * ks;
  const int nk = static_cast<int>(ks / KRowLoader<E, kBM>::kSliceElems);
  Acc<128> acc;
  {
    KRowLoader<E, kBM> la;
    la.init(static_cast<const char*>(p.dg_d) + k0 * E::kBytes, p.F, m0, n, nullptr);
    MNColLoader<E, 128> lb;
    lb.init(static_cast<const char*>(p.w_gate_t) + k0 * p.d * E::kBytes, p.d, n0, p.d, ks);
    gemm_mainloop<E, 128>(la, lb, nk, lds, acc);
  }
  {
    KRowLoader<E, kBM> la;
    la.init(static_cast<const char*>(p.du_d) + k0 * E::kBytes, p.F, m0, n, nullptr);
    MNColLoader<E, 128> lb;
    lb.init(static_cast<const char*>(p.w_up_t) + k0 * p.d * E::kBytes, p.d, n0, p.d, ks);
    gemm_mainloop<E, 128>(la, lb, nk, lds, acc, /*accumulate=*/true);
  }
  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n) continue;
      if (splits > 1) {
        float* o = p.dx_part + (static_cast<int64_t>(blockIdx.z) * p.cap + m) * p.d + n0 + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[nb * 32] = acc.c[mb][nb][r];
        continue;
      }
      const int64_t row = p.dense_rows[m];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        store_bits<E>(p.dx, row * p.d + n0 + nb * 32 + (lane & 31), round_store<E>(acc.c[mb][nb][r]).bits);
    }
}

// blockIdx.z: 0 -> dW_gate^T += dG^T x_d, 1 -> dW_up^T += dU^T x_d, 2 -> dW_down += H^T dy_d
template <class E>
__global__ __launch_bounds__(kThreads, 2) void bwd_dw_dense_kernel(BwdArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n = n_dense_of(p);
  if (n <= 0) return;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128;  // d_model columns
  const int64_t j0 = static_cast<int64_t>(blockIdx.y) * kBM;  // neurons
  const int z = blockIdx.z;
  const void* A = z == 0 ? p.dg_d : (z == 1 ? p.du_d : p.h_d);
  const void* B = z == 2 ? p.dy : p.x;
  float* out = z == 0 ? p.dw_gate_t : (z == 1 ? p.dw_up_t : p.dw_down);
  MNColLoader<E, kBM> la;
  la.init(A, p.F, j0, p.F, n);
  MNColLoader<E, 128> lb;
  lb.init(B, p.d, n0, p.d, n, p.dense_rows);
  Acc<128> acc;
  const int nk = static_cast<int>((n + MNColLoader<E, 128>::kSliceElems - 1) / MNColLoader<E, 128>::kSliceElems);
  gemm_mainloop<E, 128>(la, lb, nk, lds, acc);
  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = j0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = wrow0 + mb * 32 + acc_row(r, lane);
      if (j >= p.F) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float* o = out + j * p.d + n0 + nb * 32 + (lane & 31);
        *o += acc.c[mb][nb][r];
      }
    }
}

template <class E>
static hipError_t launch_bwd_dense_t(const BwdArgs& a, hipStream_t s) {
  const unsigned mrows = static_cast<unsigned>((a.cap + kBM - 1) / kBM);
  const size_t lds = (kBM + 128) * 128;
  hipLaunchKernelGGL((bwd_gu_kernel<E>), dim3(a.F / 64, mrows), dim3(kThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dh_kernel<E>), dim3((a.F + 127) / 128, mrows), dim3(kThreads), lds, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int splits = a.dx_splits > 1 ? a.dx_splits : 1;
  hipLaunchKernelGGL((bwd_dx_kernel<E>), dim3(a.d / 128, mrows, splits), dim3(kThreads), lds, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (splits > 1) {
    e = launch_splitk_reduce(a.dx_part, splits, a.cap, a.n_rows + 1, a.dense_rows, a.dx, a.d,
                             E::kBytes == 2 ? 1 : 0, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_dw_dense_kernel<E>), dim3(a.d / 128, (a.F + kBM - 1) / kBM, 3), dim3(kThreads), lds, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_bwd_dense(const BwdArgs& a, int dtype, hipStream_t s) {
  if (a.cap <= 0) return hipSuccess;
  return dtype == 1 ? launch_bwd_dense_t<EBf16>(a, s) : launch_bwd_dense_t<EF32>(a, s);
}

}  // namespace twell
