// Classic ELL construction, the baseline the TwELL page measures its epilogue
// packing against (page "Sakana AI and NVIDIA introduce TwELL with CUDA
// kernels...", sections "¿Cuál es el problema que TwELL resuelve?" and "¿Qué
// hace distinto a TwELL frente a ELL clásico?": converting a dense activation
// tensor to a sparse format in a separate kernel costs a launch plus a full
// write and read of that tensor, which eats the saving).
//
//   gate_dense256_kernel: the same gate GEMM as the pack kernel (256 x 256
//       core, identical K order, so g is bitwise the same) whose epilogue
//       writes ReLU(g) rounded to dtype densely, [T x d_ff];
//   ell_convert_kernel:   one wave per (row, tile) reads the tile's tile_n
//       values (lane l holds columns V*l .. V*l + V - 1, V = tile_n / 64) and
//       compacts the non-zeros in ascending column order with ballots, into
//       the same TwELL planes twell_pack writes (true count; unused slots
//       (0, +0)).
#include "gemm256.hpp"
#include "internal.hpp"

namespace twell {

template <class E>
__global__ __launch_bounds__(256, 1) void gate_dense256_kernel(ClassicArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int n_mt = static_cast<int>((p.T + kT256 - 1) / kT256);
  const int n_nt = (p.F + kT256 - 1) / kT256;
  int mt, nt;
  tile_coords_256(n_mt, n_nt, mt, nt);
  const int64_t m0 = static_cast<int64_t>(mt) * kT256, n0 = static_cast<int64_t>(nt) * kT256;
  DirectRows<E> la, lb;
  la.init(p.x, p.d, m0, p.T, nullptr);
  lb.init(p.w_gate_t, p.d, n0, p.F, nullptr);
  Acc256 acc;
  gemm256_mainloop<E>(la, lb, p.d / (128 / E::kBytes), lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wrow0 = m0 + (wave >> 1) * 128;
  const int64_t col0 = n0 + (wave & 1) * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = wrow0 + i * 32 + acc_row(r, lane);
      if (m >= p.T) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = col0 + j * 32;
        if (c >= p.F) continue;
        const float g = acc.c[i][j][r];
        store_bits<E>(p.dense, m * p.F + c, round_store<E>(g > 0.f ? g : 0.f).bits);
      }
    }
  }
}

template <class E, int V>
__global__ __launch_bounds__(256) void ell_convert_kernel(ClassicArgs p) {
  const int lane = threadIdx.x & 63;
  const int n_t = p.F / p.tile_n;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // (row, tile)
  if (unit >= p.T * n_t) return;
  const int64_t row = unit / n_t;
  const int b = static_cast<int>(unit - row * n_t);
  const int64_t base = row * p.F + static_cast<int64_t>(b) * p.tile_n + lane * V;
  uint32_t bits[V];
  int c = 0, flags = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    bits[v] = E::kBytes == 2 ? static_cast<const uint16_t*>(p.dense)[base + v]
                             : static_cast<const uint32_t*>(p.dense)[base + v];
    const bool nz = bits[v] != 0u;  // ReLU output: +0 or a positive value
    flags |= (nz ? 1 : 0) << v;
    c += nz ? 1 : 0;
  }
  int excl = 0, count = 0;
#pragma unroll
  for (int k = 1; k <= V; ++k) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(c >= k);
    excl += static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
    count += static_cast<int>(__popcll(m));
  }
  const int C = p.C;
  const int64_t rec = unit * C;
  if (lane == 0) p.count[unit] = count;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if ((flags >> v) & 1) {
      const int s = excl + __popc(flags & ((1 << v) - 1));
      if (s < C) {
        p.idx[rec + s] = static_cast<uint8_t>(lane * V + v);
        store_bits<E>(p.val, rec + s, bits[v]);
      }
    }
  }
  // slots past the stored entries: (0, +0); disjoint from the slots written above
  for (int s = lane; s < C; s += 64)
    if (s >= count) {
      p.idx[rec + s] = 0;
      store_bits<E>(p.val, rec + s, 0u);
    }
}

template <class E>
static hipError_t launch_classic_t(const ClassicArgs& a, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_dense256_kernel<E>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds256);
  if (attr != hipSuccess) return attr;
  const unsigned n_mt = static_cast<unsigned>((a.T + kT256 - 1) / kT256);
  const unsigned n_nt = static_cast<unsigned>((a.F + kT256 - 1) / kT256);
  hipLaunchKernelGGL((gate_dense256_kernel<E>), dim3(n_mt * n_nt), dim3(256), kLds256, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = a.T * (a.F / a.tile_n);
  const dim3 grid(static_cast<unsigned>((units + 3) / 4));
  if (a.tile_n == 128)
    hipLaunchKernelGGL((ell_convert_kernel<E, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((ell_convert_kernel<E, 1>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_classic_pack(const ClassicArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_classic_t<EBf16>(a, s) : launch_classic_t<EF32>(a, s);
}

}  // namespace twell
