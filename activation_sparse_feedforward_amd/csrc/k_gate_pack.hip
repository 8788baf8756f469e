// Gate GEMM with a ReLU + TwELL-packing epilogue, one dispatch.
//
// Follows the TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA
// kernels...", section "¿Qué hace distinto a TwELL frente a ELL clásico?"):
// the sparse format is produced inside the epilogue of the gate matmul, the
// activation columns are cut into tiles equal to the matmul's N tile, and the
// non-zeros are packed locally per tile.  Here the N tile of a workgroup IS
// one TwELL tile (BN = T_n) and every wave owns whole rows of it, so each
// (row, tile) is compacted straight from the MFMA accumulators: a wavefront
// ballot per 32-column block gives the non-zero mask of two rows at once, and
// popcounts of the masks give every non-zero its slot in ascending column
// order -- no atomics, no LDS round trip, no dense store of ReLU(g).
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

template <class E, int BN>
__global__ __launch_bounds__(kThreads, 2) void gate_pack_kernel(PackArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int b = blockIdx.x;                       // TwELL tile index == N tile
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int n_t = p.F / BN;

  KRowLoader<E, kBM> la;
  KRowLoader<E, BN> lb;
  la.init(p.x, p.d, m0, p.T, nullptr);
  lb.init(p.w_gate_t, p.d, static_cast<int64_t>(b) * BN, p.F, nullptr);
  Acc<BN> acc;
  gemm_mainloop<E, BN>(la, lb, p.d / KRowLoader<E, kBM>::kSliceElems, lds, acc);

  constexpr int kWN = BN / 32;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, li = lane & 31;
  const int64_t wrow0 = m0 + (threadIdx.x >> 6) * 64;
  const int C = p.C;
  uint32_t ovf = 0, nnz = 0;

#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = wrow0 + mb * 32 + acc_row(r, lane);
      const bool valid = row < p.T;
      uint32_t bits[kWN];
      uint32_t mh[kWN];
      bool nz[kWN];
#pragma unroll
      for (int nb = 0; nb < kWN; ++nb) {
        const float g = acc.c[mb][nb][r];
        const Rounded<E> a = round_store<E>(g > 0.f ? g : 0.f);
        bits[nb] = a.bits;
        nz[nb] = a.bits != 0u;
        const uint64_t m = __ballot(nz[nb]);
        mh[nb] = half ? static_cast<uint32_t>(m >> 32) : static_cast<uint32_t>(m);
      }
      if (!valid) continue;
      const int64_t rt = row * n_t + b;  // (row, tile) record index
      int pre = 0;
#pragma unroll
      for (int nb = 0; nb < kWN; ++nb) {
        if (nz[nb]) {
          const int s = pre + __popc(mh[nb] & ((1u << li) - 1u));
          if (s < C) {
            p.idx[rt * C + s] = static_cast<uint8_t>(nb * 32 + li);
            store_bits<E>(p.val, rt * C + s, bits[nb]);
          }
        }
        pre += __popc(mh[nb]);
      }
      for (int s = li; s < C; s += 32) {
        if (s >= pre) {
          p.idx[rt * C + s] = 0;
          store_bits<E>(p.val, rt * C + s, 0u);
        }
      }
      if (li == 0) {
        p.count[rt] = pre;
        ovf += pre > C ? 1u : 0u;
        nnz += static_cast<uint32_t>(pre);
      }
      if (p.gate_dbg) {
#pragma unroll
        for (int nb = 0; nb < kWN; ++nb)
          store_bits<E>(p.gate_dbg, row * p.F + static_cast<int64_t>(b) * BN + nb * 32 + li, bits[nb]);
      }
    }
  }
  if (p.stats) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      ovf += __shfl_xor(ovf, o);
      nnz += __shfl_xor(nnz, o);
    }
    if (lane == 0) {
      if (ovf) atomicAdd(p.stats + 0, static_cast<unsigned long long>(ovf));
      if (nnz) atomicAdd(p.stats + 1, static_cast<unsigned long long>(nnz));
    }
  }
}

template <class E, int BN>
static hipError_t launch_pack_t(const PackArgs& a, hipStream_t s) {
  dim3 grid(a.F / BN, static_cast<unsigned>((a.T + kBM - 1) / kBM));
  const size_t lds = (kBM + BN) * 128;
  hipLaunchKernelGGL((gate_pack_kernel<E, BN>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gate_pack(const PackArgs& a, int dtype, hipStream_t s) {
  if (dtype == 1) return a.tile_n == 128 ? launch_pack_t<EBf16, 128>(a, s) : launch_pack_t<EBf16, 64>(a, s);
  return a.tile_n == 128 ? launch_pack_t<EF32, 128>(a, s) : launch_pack_t<EF32, 64>(a, s);
}

}  // namespace twell
