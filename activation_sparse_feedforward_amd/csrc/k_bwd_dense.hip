// Backward of the rows the hybrid format sent to the dense fallback, on MFMA.
//
// Same loss as the sparse backward (sum(y*dy) + l1 sum|h|, h = ReLU(g)*u); for
// these few rows everything is dense, so it is GEMM launches over the
// gathered rows (n_dense is read on the device; workgroups past it exit):
//   gue: g, u, e = x_d W_gate, x_d W_up, dy_d W_down^T (recomputed; one launch,
//        blockIdx.z picks the product; fp32 into the workspace)
//   act: elementwise dh = e + l1 sign(h), du = dh a, dg = dh u [g>0]
//        -> dG, dU, H (dtype) in the workspace
//   dx:  dx_d = dG W_gate^T... in the stored layout: dx[t,k] = sum_j dG[m,j] W_gate^T[j,k]
//        + dU[m,j] W_up^T[j,k]; two K passes into one accumulator, rows scattered
//   dw:  dW_gate^T += dG^T x_d, dW_up^T += dU^T x_d, dW_down += H^T dy_d
//        (both operands MN-contiguous, K = n_dense, fp32 read-modify-write on
//        top of the sparse rows' contribution written before)
// The dense rows are few (n_dense ~ 250 of 16384 at the training workload), so
// the three products share one launch of 3 x d_ff/64 workgroups instead of
// leaving most of the chip idle in two smaller ones.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

namespace {
__device__ __forceinline__ int64_t n_dense_of(const BwdArgs& p) { return static_cast<int64_t>(p.n_rows[1]); }

// K slices [0, nk) from base b0, [nk, 2 nk) from base b1, through one loader.
template <class L>
struct TwoSource {
  L& l;
  const char* b0;
  const char* b1;
  int nk;
  __device__ __forceinline__ void load(int kt) {
    l.base = kt < nk ? b0 : b1;
    l.load(kt < nk ? kt : kt - nk);
  }
  __device__ __forceinline__ void store(char* lds, int row_base) const { l.store(lds, row_base); }
};
}  // namespace

// blockIdx.z: 0 -> g = x_d W_gate, 1 -> u = x_d W_up, 2 -> e = dy_d W_down^T
template <class E>
__global__ __launch_bounds__(kThreads, 2) void bwd_gue_kernel(BwdArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t n = n_dense_of(p);
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  if (m0 >= n) return;
  const int z = blockIdx.z;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
  KRowLoader<E, kBM> la;
  la.init(z == 2 ? p.dy : p.x, p.d, m0, n, p.dense_rows);
  KRowLoader<E, 64> lb;
  lb.init(z == 0 ? p.w_gate_t : (z == 1 ? p.w_up_t : p.w_down), p.d, j0, p.F, nullptr);
  Acc<64> acc;
  gemm_mainloop<E, 64>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);
  float* out = z == 0 ? p.g_d : (z == 1 ? p.u_d : p.e_d);
  const int lane = threadIdx.x & 63;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + mb * 32 + acc_row(r, lane);
      if (m >= n) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) out[m * p.F + j0 + nb * 32 + (lane & 31)] = acc.c[mb][nb][r];
    }
}

// Four consecutive neurons of one dense row per thread.
template <class E>
__global__ __launch_bounds__(256) void bwd_dense_act_kernel(BwdArgs p) {
  const int64_t n = n_dense_of(p);
  const int64_t q = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (q >= n * p.F) return;  // F is a multiple of 64, so the 4 elements share a row
  const float4 g4 = *reinterpret_cast<const float4*>(p.g_d + q);
  const float4 u4 = *reinterpret_cast<const float4*>(p.u_d + q);
  const float4 e4 = *reinterpret_cast<const float4*>(p.e_d + q);
  const float gs[4] = {g4.x, g4.y, g4.z, g4.w}, us[4] = {u4.x, u4.y, u4.z, u4.w}, es[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g = gs[i], u = us[i];
    const float a = g > 0.f ? g : 0.f;
    const float h = a * u;
    const float sg = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
    const float dh = es[i] + p.l1 * sg;
    store_bits<E>(p.du_d, q + i, round_store<E>(dh * a).bits);
    store_bits<E>(p.dg_d, q + i, round_store<E>(g > 0.f ? dh * u : 0.f).bits);
    store_bits<E>(p.h_d, q + i, round_store<E>(h).bits);
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
  // one main loop over 2 nk slices: (dG, W_gate^T) then (dU, W_up^T), the
  // same loaders re-pointed (two inlined loops spilled the accumulators)
  KRowLoader<E, kBM> la;
  la.init(static_cast<const char*>(p.dg_d) + k0 * E::kBytes, p.F, m0, n, nullptr);
  MNColLoader<E, 128> lb;
  lb.init(static_cast<const char*>(p.w_gate_t) + k0 * p.d * E::kBytes, p.d, n0, p.d, ks);
  TwoSource<KRowLoader<E, kBM>> sa{la, la.base, static_cast<const char*>(p.du_d) + k0 * E::kBytes, nk};
  TwoSource<MNColLoader<E, 128>> sb{lb, lb.base, static_cast<const char*>(p.w_up_t) + k0 * p.d * E::kBytes, nk};
  Acc<128> acc;
  gemm_mainloop<E, 128>(sa, sb, 2 * nk, lds, acc);
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

// blockIdx.z: 0 -> dW_gate^T = dG^T x_d, 1 -> dW_up^T = dU^T x_d, 2 -> dW_down = H^T dy_d
// (stored; the ELL rows' per-neuron pass, launched after this one, adds these
// rows to its own sums).  With no dense rows nothing is written.
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
        out[j * p.d + n0 + nb * 32 + (lane & 31)] = acc.c[mb][nb][r];
      }
    }
}

template <class E>
static hipError_t launch_bwd_dense_t(const BwdArgs& a, hipStream_t s) {
  const unsigned mrows = static_cast<unsigned>((a.cap + kBM - 1) / kBM);
  const size_t lds = (kBM + 128) * 128;
  hipLaunchKernelGGL((bwd_gue_kernel<E>), dim3(a.F / 64, mrows, 3), dim3(kThreads), (kBM + 64) * 128, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t quads = a.cap * a.F / 4;
  hipLaunchKernelGGL((bwd_dense_act_kernel<E>), dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), 0, s, a);
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
