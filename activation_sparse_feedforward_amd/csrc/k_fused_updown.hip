// Fused TwELL up + down projection, one dispatch.
//
// Follows the TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA
// kernels...", section "¿Qué hace distinto a TwELL frente a ELL clásico?"):
// one fused kernel reads the TwELL activations and runs the up and down
// projections together, and the intermediate never goes to global memory.
//
// Design (gfx950, wave64): one wavefront per token row t.  x[t] and the fp32
// accumulator of y[t] live in VGPRs, spread over the 64 lanes in 16-byte
// chunks.  The wave first turns the row's TwELL records into a compact list of
// (neuron j, activation a) in LDS (one lane per tile, a wave prefix sum of the
// clamped counts), then walks the list in ascending j, U neurons at a time:
//   u_j = x[t] . W_up^T[j]   (coalesced 16-byte loads of the contiguous row,
//                             lane partial dots, DPP + shuffle wave reduction)
//   y[t] += (a_j * u_j) * W_down[j]   (coalesced 16-byte loads, fp32 FMAs)
// and finally writes y[t] once.  The walk is bound by the gather of the two
// weight rows per active neuron, which are served mostly from the MALL.
#include "common.hpp"
#include "internal.hpp"

namespace twell {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kListCap = 1024;  // list entries per wave and per chunk of tiles

// Neurons in flight per wave: enough 16-byte loads outstanding to cover the
// gather latency, without spilling at the widest rows.
template <int NV> constexpr int neurons_in_flight() { return NV <= 1 ? 8 : (NV <= 4 ? 4 : 2); }

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror: combine the two quads of each 8
  v = dpp_add<0x140>(v);  // row_mirror: combine the two 8-lane halves of each row of 16
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <class E> struct Vec;  // 16 bytes of storage as fp32 values
template <> struct Vec<EBf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4_t& r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4_t pack(const float* f) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
    return r;
  }
};
template <> struct Vec<EF32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t& r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
  __device__ __forceinline__ static u32x4_t pack(const float* f) {
    return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

// Inclusive prefix sum over the wave (Hillis-Steele with shuffles); small and
// only run once per 64 tiles.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

}  // namespace

// NV = 16-byte vectors per lane per row: d_model = NV * 64 * Vec<E>::N.
template <class E, int NV>
__global__ __launch_bounds__(kWavesPerBlock * kWave, 2) void fused_updown_kernel(FusedArgs p) {
  constexpr int kN = Vec<E>::N;
  constexpr int kU = neurons_in_flight<NV>();
  __shared__ int2 list_all[kWavesPerBlock][kListCap];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t i_row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.T;
  if (i_row >= n_rows) return;  // whole wave exits together; no block barrier below
  const int64_t t = p.rows ? static_cast<int64_t>(p.rows[i_row]) : i_row;
  int2* list = list_all[wave];
  const int d = p.d, C = p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;

  // x[t] (kept in storage form) and the fp32 y accumulator, lane-strided 16-byte chunks
  u32x4_t xs[NV];
  float yf[NV][kN];
  {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      xs[v] = xr[v * kWave + lane];
#pragma unroll
      for (int i = 0; i < kN; ++i) yf[v][i] = 0.f;
    }
  }

  const int chunk_tiles = min(kWave, kListCap / C);
  for (int b0 = 0; b0 < n_t; b0 += chunk_tiles) {
    // ---- build the (j, a) list of this chunk of tiles, ascending j
    const int b = b0 + lane;
    int cnt = 0;
    // counts are clamped to [0, C] and tile-local indices masked to the tile
    // width (a power of two), so even a corrupted TwELL stays in bounds
    if (lane < chunk_tiles && b < n_t) cnt = max(0, min(p.count[t * n_t + b], C));
    const int incl = wave_incl_scan(cnt, lane);
    const int total = __shfl(incl, 63);
    const int off = incl - cnt;
    if (cnt > 0) {
      const int64_t rec = (t * n_t + b) * C;
      for (int s = 0; s < cnt; ++s) {
        const int j = b * tile_n + (p.idx[rec + s] & (tile_n - 1));
        const float a = load_elem<E>(p.val, rec + s);
        list[off + s] = make_int2(j, __float_as_int(a));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- walk the list, kU neurons at a time
    for (int e0 = 0; e0 < total; e0 += kU) {
      int jj[kU];
      float aa[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int e = min(e0 + q, total - 1);
        const int2 ent = list[e];
        jj[q] = __builtin_amdgcn_readfirstlane(ent.x);
        aa[q] = (e0 + q < total) ? __int_as_float(__builtin_amdgcn_readfirstlane(ent.y)) : 0.f;
      }
      const int nq = min(kU, total - e0);  // wave-uniform
      u32x4_t wu[kU][NV], wd[kU][NV];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const u32x4_t* ur =
            reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + int64_t(jj[q]) * d * E::kBytes);
        const u32x4_t* dr =
            reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + int64_t(jj[q]) * d * E::kBytes);
        if (q < nq) {
#pragma unroll
          for (int v = 0; v < NV; ++v) wu[q][v] = ur[v * kWave + lane];
#pragma unroll
          for (int v = 0; v < NV; ++v) wd[q][v] = dr[v * kWave + lane];
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) wu[q][v] = wd[q][v] = u32x4_t{0, 0, 0, 0};
        }
      }
      float hq[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        float part = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float w[kN], xv[kN];
          Vec<E>::unpack(wu[q][v], w);
          Vec<E>::unpack(xs[v], xv);
#pragma unroll
          for (int i = 0; i < kN; ++i) part = fmaf(xv[i], w[i], part);
        }
        hq[q] = part;
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) hq[q] = aa[q] * wave_sum(hq[q]);
#pragma unroll
      for (int q = 0; q < kU; ++q) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float w[kN];
          Vec<E>::unpack(wd[q][v], w);
#pragma unroll
          for (int i = 0; i < kN; ++i) yf[v][i] = fmaf(hq[q], w[i], yf[v][i]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  u32x4_t* yr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.y) + t * d * E::kBytes);
#pragma unroll
  for (int v = 0; v < NV; ++v) yr[v * kWave + lane] = Vec<E>::pack(yf[v]);
}

template <class E, int NV>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.T + kWavesPerBlock - 1) / kWavesPerBlock));
  hipLaunchKernelGGL((fused_updown_kernel<E, NV>), grid, dim3(kWavesPerBlock * kWave), 0, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fused_e(const FusedArgs& a, hipStream_t s) {
  const int nv = a.d / (kWave * Vec<E>::N);
  switch (nv) {
    case 1: return launch_fused_t<E, 1>(a, s);
    case 2: return launch_fused_t<E, 2>(a, s);
    case 3: return launch_fused_t<E, 3>(a, s);
    case 4: return launch_fused_t<E, 4>(a, s);
    case 5: return launch_fused_t<E, 5>(a, s);
    case 6: return launch_fused_t<E, 6>(a, s);
    case 7: return launch_fused_t<E, 7>(a, s);
    case 8: return launch_fused_t<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused_updown(const FusedArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_fused_e<EBf16>(a, s) : launch_fused_e<EF32>(a, s);
}

}  // namespace twell
