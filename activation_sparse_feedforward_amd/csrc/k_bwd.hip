// Backward of the TwELL FFN on the rows served from TwELL (the ELL rows of the
// hybrid format), reusing the forward's TwELL indices.
//
// Loss (reading of the training recipe on the TwELL page "Sakana AI and NVIDIA
// introduce TwELL with CUDA kernels...", section "Receta de entrenamiento":
// ReLU gate plus an L1 penalty on the hidden activations):
//     L = sum(y * dy) + l1 * sum|h|,   h = ReLU(g) * u.
// Only active (row, neuron) pairs have non-zero gradients (ReLU' = 0 and
// h = 0 elsewhere), so every gradient is a sum over the stored TwELL slots:
//     u = x[t].W_up^T[j],  h = a u,  dh = dy[t].W_down[j] + l1 sign(h)
//     du = dh a,  dg = dh u
//     dx[t]       += dg W_gate^T[j] + du W_up^T[j]           (token-major)
//     dW_gate^T[j] += dg x[t],  dW_up^T[j] += du x[t],  dW_down[j] += h dy[t]
//                                                            (neuron-major)
// TwELL is token-major, so the pairs are transposed to neuron-major order by a
// counting sort that keeps ascending t inside each neuron (deterministic dW):
//   hist     per block of 64 ELL rows, LDS histogram of neuron ids
//   colscan  per neuron, exclusive scan over the blocks
//   nscan    exclusive scan over neurons -> start of each neuron's pair list
//   pos      per block, rows in order, one LDS cursor per neuron -> the
//            destination of every (row, slot) pair (within one row every
//            neuron occurs at most once, so a wave's lanes never collide)
//   totals   per row, the sum of its counts; the ELL rows are then split into
//            light rows and at most heavy_cap heavy ones (row total >
//            max(2 C, 2 x mean)), as in the hybrid forward
//   token    light rows: 16-wave workgroups walking the tiles in lockstep
//            (x[t], dy[t] in LDS, one row per wave; the weight rows of the
//            current tiles are shared through L2); heavy rows: one wave per
//            (row, tile range) with fp32 partial dx reduced in a fixed order;
//            both write dx[t] and the pair records {t, dg, du, h}
//   dw       one wave per neuron: walks its pairs in ascending t, fp32 rows
//            of the three weight gradients in VGPRs, written once.
#include "common.hpp"
#include "internal.hpp"

namespace twell {

namespace {

constexpr int kBlkRows = 64;         // ELL rows per counting-sort block
constexpr int kNeuronChunk = 8192;   // neurons per LDS histogram / cursor table
constexpr int kTokWaves = 4;
constexpr int kTokListCap = 512;

__device__ __forceinline__ int64_t n_ell_of(const BwdArgs& p) { return static_cast<int64_t>(p.n_rows[0]); }

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

template <class E> struct VecB;
template <> struct VecB<EBf16> {
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
template <> struct VecB<EF32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t& r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
  __device__ __forceinline__ static u32x4_t pack(const float* f) {
    return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Per-lane partial dot product of two rows held as NV 16-byte vectors; bf16
// pairs go through v_dot2c_f32_bf16 (fp32 accumulate) without unpacking, in
// four interleaved partial sums.  (The 16-byte vector is bit-cast whole to
// bf16x8 before taking pairs: casting an element of the 32-bit vector directly
// was compiled to always read element 0.)
template <class E, int NV>
__device__ __forceinline__ float row_dot(const u32x4_t* w, const u32x4_t* x) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if constexpr (E::kBytes == 2) {
      const bf16x8_t wh = __builtin_bit_cast(bf16x8_t, w[v]);
      const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, x[v]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{wh[2 * i], wh[2 * i + 1]},
                                                 bf16x2_t{xh[2 * i], xh[2 * i + 1]}, acc[i], false);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(__uint_as_float(w[v][i]), __uint_as_float(x[v][i]), acc[i]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// One 16-byte piece of row_dot, accumulated into the same four chains.
template <class E>
__device__ __forceinline__ void row_dot_piece(const u32x4_t& w, const u32x4_t& x, float (&acc)[4]) {
  if constexpr (E::kBytes == 2) {
    const bf16x8_t wh = __builtin_bit_cast(bf16x8_t, w);
    const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{wh[2 * i], wh[2 * i + 1]}, bf16x2_t{xh[2 * i], xh[2 * i + 1]},
                                               acc[i], false);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(__uint_as_float(w[i]), __uint_as_float(x[i]), acc[i]);
  }
}

}  // namespace

// ---------------------------------------------------------------- hist
__global__ __launch_bounds__(256) void bwd_hist_kernel(BwdArgs p) {
  __shared__ int hist[kNeuronChunk];
  const int blk = blockIdx.x;
  const int j0 = blockIdx.y * kNeuronChunk;
  const int nj = min(kNeuronChunk, p.F - j0);
  for (int j = threadIdx.x; j < nj; j += 256) hist[j] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_t = p.F / p.tile_n;
  const int64_t n_ell = n_ell_of(p);
  for (int r = wave; r < kBlkRows; r += 4) {
    const int64_t i = static_cast<int64_t>(blk) * kBlkRows + r;
    if (i >= n_ell) break;
    const int64_t t = p.ell_rows[i];
    for (int b = lane; b < n_t; b += 64) {
      const int cnt = max(0, min(p.count[t * n_t + b], p.C));
      const int64_t rec = (t * n_t + b) * p.C;
      for (int s = 0; s < cnt; ++s) {
        const int j = b * p.tile_n + (p.idx[rec + s] & (p.tile_n - 1)) - j0;
        if (j >= 0 && j < nj) atomicAdd(&hist[j], 1);
      }
    }
  }
  __syncthreads();
  int32_t* out = p.blk_hist + static_cast<int64_t>(blk) * p.F + j0;
  for (int j = threadIdx.x; j < nj; j += 256) out[j] = hist[j];
}

// ---------------------------------------------------------------- column scan
__global__ __launch_bounds__(256) void bwd_colscan_kernel(BwdArgs p, int nblk) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= p.F) return;
  int run = 0;
  for (int b = 0; b < nblk; ++b) {
    int32_t* h = p.blk_hist + static_cast<int64_t>(b) * p.F + j;
    const int c = *h;
    *h = run;
    run += c;
  }
  p.neuron_off[j] = run;  // per-neuron total; turned into offsets by nscan
}

// ---------------------------------------------------------------- neuron scan (one block)
__global__ __launch_bounds__(1024) void bwd_nscan_kernel(BwdArgs p) {
  __shared__ int wpre[16];
  __shared__ int carry_s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < p.F; base += 1024) {
    const int j = base + threadIdx.x;
    const int v = j < p.F ? p.neuron_off[j] : 0;
    const int incl = wave_incl_scan(v, lane);
    if (lane == 63) wpre[wave] = incl;
    __syncthreads();
    int off = carry_s;
    for (int w = 0; w < wave; ++w) off += wpre[w];
    if (j < p.F) p.neuron_off[j] = off + incl - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry_s = off + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) p.neuron_off[p.F] = carry_s;
}

// ---------------------------------------------------------------- positions (one wave per block)
__global__ __launch_bounds__(64) void bwd_pos_kernel(BwdArgs p) {
  __shared__ int cursor[kNeuronChunk];
  const int blk = blockIdx.x;
  const int j0 = blockIdx.y * kNeuronChunk;
  const int nj = min(kNeuronChunk, p.F - j0);
  const int lane = threadIdx.x;
  const int32_t* hb = p.blk_hist + static_cast<int64_t>(blk) * p.F + j0;
  for (int j = lane; j < nj; j += 64) cursor[j] = p.neuron_off[j0 + j] + hb[j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int n_t = p.F / p.tile_n;
  const int64_t n_ell = n_ell_of(p);
  for (int r = 0; r < kBlkRows; ++r) {
    const int64_t i = static_cast<int64_t>(blk) * kBlkRows + r;
    if (i >= n_ell) break;
    const int64_t t = p.ell_rows[i];
    for (int b0 = 0; b0 < n_t; b0 += 64) {
      const int b = b0 + lane;
      const int cnt = b < n_t ? max(0, min(p.count[t * n_t + b], p.C)) : 0;
      const int maxc = wave_max(cnt);
      const int64_t rec = (t * n_t + b) * p.C;
      for (int s = 0; s < maxc; ++s) {
        if (s < cnt) {
          const int j = b * p.tile_n + (p.idx[rec + s] & (p.tile_n - 1)) - j0;
          if (j >= 0 && j < nj) {
            const int q = cursor[j];
            cursor[j] = q + 1;
            p.pos[rec + s] = q;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
}

// ---------------------------------------------------------------- token pass
// One wave per ELL row (SPLIT = false: every ELL row; used where the lockstep
// kernel does not fit), or per (heavy row, tile range) with fp32 partial dx
// written to dx_hpart[range][i][:] (SPLIT = true).
template <class E, int NV, bool SPLIT>
__global__ __launch_bounds__(kTokWaves * kWave, 2) void bwd_token_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  constexpr int kU = NV <= 2 ? 4 : 2;
  __shared__ int4 list_all[kTokWaves][kTokListCap];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kTokWaves + wave;
  const int d = p.d, C = p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  int64_t i_row = unit;
  int grp = 0, b_begin = 0, b_end = n_t;
  int64_t t;
  if constexpr (SPLIT) {
    const int64_t n_heavy = min(static_cast<int64_t>(p.split_n[1]), p.heavy_cap);
    if (unit >= n_heavy * p.groups) return;
    i_row = unit / p.groups;
    grp = static_cast<int>(unit - i_row * p.groups);
    const int tg = (n_t + p.groups - 1) / p.groups;
    b_begin = min(n_t, grp * tg);
    b_end = min(n_t, b_begin + tg);
    t = p.heavy_rows[i_row];
  } else {
    if (i_row >= n_ell_of(p)) return;
    t = p.ell_rows[i_row];
  }
  int4* list = list_all[wave];

  u32x4_t xs[NV], dys[NV];
  float dxf[NV][kN];
  {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
    const u32x4_t* yr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.dy) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      xs[v] = xr[v * kWave + lane];
      dys[v] = yr[v * kWave + lane];
#pragma unroll
      for (int i = 0; i < kN; ++i) dxf[v][i] = 0.f;
    }
  }
  const int chunk_tiles = min(kWave, kTokListCap / C);
  for (int b0 = b_begin; b0 < b_end; b0 += chunk_tiles) {
    const int b = b0 + lane;
    int cnt = 0;
    if (lane < chunk_tiles && b < b_end) cnt = max(0, min(p.count[t * n_t + b], C));
    const int incl = wave_incl_scan(cnt, lane);
    const int total = __shfl(incl, 63);
    const int off = incl - cnt;
    if (cnt > 0) {
      const int64_t rec = (t * n_t + b) * C;
      for (int s = 0; s < cnt; ++s) {
        const int j = b * tile_n + (p.idx[rec + s] & (tile_n - 1));
        const float a = load_elem<E>(p.val, rec + s);
        list[off + s] = make_int4(j, __float_as_int(a), p.pos[rec + s], 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    for (int e0 = 0; e0 < total; e0 += kU) {
      const int nq = min(kU, total - e0);
      int jj[kU], pp[kU];
      float aa[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int4 ent = list[min(e0 + q, total - 1)];
        jj[q] = __builtin_amdgcn_readfirstlane(ent.x);
        aa[q] = __int_as_float(__builtin_amdgcn_readfirstlane(ent.y));
        pp[q] = __builtin_amdgcn_readfirstlane(ent.z);
      }
      u32x4_t wu[kU][NV], wd[kU][NV], wg[kU][NV];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int64_t ro = int64_t(jj[q]) * d * E::kBytes;
        const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
        const u32x4_t* dr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + ro);
        const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_gate_t) + ro);
        if (q < nq) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            wu[q][v] = ur[v * kWave + lane];
            wd[q][v] = dr[v * kWave + lane];
            wg[q][v] = gr[v * kWave + lane];
          }
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) wu[q][v] = wd[q][v] = wg[q][v] = u32x4_t{0, 0, 0, 0};
        }
      }
      float uu[kU], ee[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        float pu = 0.f, pe = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float w1[kN], w2[kN], xv[kN], yv[kN];
          VecB<E>::unpack(wu[q][v], w1);
          VecB<E>::unpack(wd[q][v], w2);
          VecB<E>::unpack(xs[v], xv);
          VecB<E>::unpack(dys[v], yv);
#pragma unroll
          for (int i = 0; i < kN; ++i) {
            pu = fmaf(xv[i], w1[i], pu);
            pe = fmaf(yv[i], w2[i], pe);
          }
        }
        uu[q] = wave_sum(pu);
        ee[q] = wave_sum(pe);
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const float a = q < nq ? aa[q] : 0.f;
        const float h = a * uu[q];
        const float sg = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
        const float dh = ee[q] + p.l1 * sg;
        const float du = dh * a;
        const float dg = q < nq ? dh * uu[q] : 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          float w1[kN], w3[kN];
          VecB<E>::unpack(wu[q][v], w1);
          VecB<E>::unpack(wg[q][v], w3);
#pragma unroll
          for (int i = 0; i < kN; ++i) dxf[v][i] = fmaf(dg, w3[i], fmaf(du, w1[i], dxf[v][i]));
        }
        if (q < nq && lane == 0)
          p.recs[pp[q]] = make_float4(__int_as_float(static_cast<int>(t)), dg, du, h);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if constexpr (SPLIT) {
    float* o = p.dx_hpart + (static_cast<int64_t>(grp) * p.heavy_cap + i_row) * d;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < kN; i += 4)
        *reinterpret_cast<float4*>(o + (v * kWave + lane) * kN + i) =
            make_float4(dxf[v][i], dxf[v][i + 1], dxf[v][i + 2], dxf[v][i + 3]);
  } else {
    u32x4_t* dxr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dx) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) dxr[v * kWave + lane] = VecB<E>::pack(dxf[v]);
  }
}

// ---------------------------------------------------------------- token pass, lockstep (light rows)
// 16 waves, one light row each; x[t] and dy[t] sit in LDS, the fp32 dx row in
// VGPRs.  Every chunk of tiles starts with a workgroup barrier, so all
// resident workgroups sweep the neurons in roughly the same order and the
// weight rows (three per active pair) are reused from L2.  The two dot
// products per pair use packed bf16 pairs (row_dot), so the rounding of u and
// dh differs in the last bits from bwd_token_kernel's unpacked fp32 sums.
constexpr int kSyncWavesB = 16;
constexpr int kSyncListB = 96;  // {j, a, pos} entries per wave per chunk

template <int NV>
constexpr size_t bwd_sync_lds_bytes() {
  return static_cast<size_t>(kSyncWavesB) * 2 * NV * kWave * 16 + kSyncWavesB * kSyncListB * 16;
}

template <class E, int NV, int kC>
__global__ __launch_bounds__(kSyncWavesB * kWave) void bwd_token_sync_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  constexpr int kRowVec = NV * kWave;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4_t* xw = reinterpret_cast<u32x4_t*>(smem) + wave * kRowVec;
  u32x4_t* yw = reinterpret_cast<u32x4_t*>(smem) + (kSyncWavesB + wave) * kRowVec;
  int4* list = reinterpret_cast<int4*>(smem + kSyncWavesB * 2 * kRowVec * 16) + wave * kSyncListB;
  const int d = p.d, C = kC > 0 ? kC : p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  const int64_t i_row = static_cast<int64_t>(blockIdx.x) * kSyncWavesB + wave;
  const bool act = i_row < static_cast<int64_t>(p.split_n[0]);  // idle waves still meet every barrier
  // wave-uniform: the token row stays in scalar registers
  const int64_t t = act ? static_cast<int64_t>(__builtin_amdgcn_readfirstlane(p.light_rows[i_row])) : 0;
  float dxf[NV][kN];
  {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
    const u32x4_t* yr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.dy) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      // x, dy, the counts / indices and dx are touched once: non-temporal
      // accesses keep them from pushing the shared weight rows out of L2
      xw[v * kWave + lane] = act ? __builtin_nontemporal_load(xr + v * kWave + lane) : u32x4_t{0, 0, 0, 0};
      yw[v * kWave + lane] = act ? __builtin_nontemporal_load(yr + v * kWave + lane) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kN; ++i) dxf[v][i] = 0.f;
    }
  }
  const int chunk_tiles = max(1, min(kWave, kSyncListB / C));
  // C = 16: the builder lanes load the next chunk's counts and 16 index bytes
  // while the current chunk's entries are processed; an entry carries its
  // slot position, from which its value and record position are loaded beside
  // the weight rows.
  int pf_cnt = 0;
  u32x4_t pf_idx{0, 0, 0, 0};
  auto prefetch = [&](int b0) {
    const int b = b0 + lane;
    pf_cnt = 0;
    if (act && lane < chunk_tiles && b < n_t) {
      const int64_t rec = t * n_t + b;
      pf_cnt = __builtin_nontemporal_load(p.count + rec);
      pf_idx = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.idx + rec * 16));
    }
  };
  if constexpr (kC == 16) prefetch(0);
  for (int b0 = 0; b0 < n_t; b0 += chunk_tiles) {
    __syncthreads();
    const int b = b0 + lane;
    int total;
    if constexpr (kC == 16) {
      const int cnt = max(0, min(pf_cnt, 16));
      const u32x4_t ix = pf_idx;
      const int incl = wave_incl_scan(cnt, lane);
      total = min(__shfl(incl, 63), kSyncListB);
      const int off = incl - cnt;
      const int spos = static_cast<int>((t * n_t + b) * 16);
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        if (s2 < cnt && off + s2 < kSyncListB) {
          const int j = b * tile_n + (static_cast<int>((ix[s2 >> 2] >> (8 * (s2 & 3))) & 0xffu) & (tile_n - 1));
          list[off + s2] = make_int4(j, spos + s2, 0, 0);
        }
      }
      if (b0 + chunk_tiles < n_t) prefetch(b0 + chunk_tiles);
    } else {
      int cnt = 0;
      if (act && lane < chunk_tiles && b < n_t) cnt = max(0, min(p.count[t * n_t + b], C));
      const int incl = wave_incl_scan(cnt, lane);
      total = min(__shfl(incl, 63), kSyncListB);
      const int off = incl - cnt;
      if (cnt > 0) {
        const int64_t rec = (t * n_t + b) * C;
        // off + cnt <= chunk_tiles * C <= kSyncListB
        for (int s2 = 0; s2 < cnt && off + s2 < kSyncListB; ++s2) {
          const int j = b * tile_n + (p.idx[rec + s2] & (tile_n - 1));
          list[off + s2] = make_int4(j, __float_as_int(load_elem<E>(p.val, rec + s2)), p.pos[rec + s2], 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e = 0; e < total; ++e) {
      const int4 ent = list[e];
      const int j = __builtin_amdgcn_readfirstlane(ent.x);
      float a;
      int pp;
      if constexpr (kC == 16) {
        const int sp = __builtin_amdgcn_readfirstlane(ent.y);
        a = load_elem<E>(p.val, sp);
        pp = p.pos[sp];
      } else {
        a = __int_as_float(__builtin_amdgcn_readfirstlane(ent.y));
        pp = __builtin_amdgcn_readfirstlane(ent.z);
      }
      const int64_t ro = int64_t(j) * d * E::kBytes;
      const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
      const u32x4_t* dr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + ro);
      const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_gate_t) + ro);
      u32x4_t wu[NV], wd[NV], wg[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        wu[v] = ur[v * kWave + lane];
        wd[v] = dr[v * kWave + lane];
        wg[v] = gr[v * kWave + lane];
      }
      // x and dy come from LDS one 16-byte piece at a time (fewer live VGPRs)
      float au[4] = {0.f, 0.f, 0.f, 0.f}, ae[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4_t xv = xw[v * kWave + lane];
        row_dot_piece<E>(wu[v], xv, au);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4_t yv = yw[v * kWave + lane];
        row_dot_piece<E>(wd[v], yv, ae);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float pu = (au[0] + au[1]) + (au[2] + au[3]);
      const float pe = (ae[0] + ae[1]) + (ae[2] + ae[3]);
      const float u = wave_sum(pu), ee = wave_sum(pe);
      const float h = a * u;
      const float sg = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
      const float dh = ee + p.l1 * sg;
      const float du = dh * a;
      const float dg = dh * u;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float w1[kN], w3[kN];
        VecB<E>::unpack(wu[v], w1);
        VecB<E>::unpack(wg[v], w3);
#pragma unroll
        for (int i = 0; i < kN; ++i) dxf[v][i] = fmaf(dg, w3[i], fmaf(du, w1[i], dxf[v][i]));
      }
      if (lane == 0) p.recs[pp] = make_float4(__int_as_float(static_cast<int>(t)), dg, du, h);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (act) {
    u32x4_t* dxr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dx) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(VecB<E>::pack(dxf[v]), dxr + v * kWave + lane);
  }
}

template <class E, int NV, int kC>
static hipError_t launch_bwd_sync_c(const BwdArgs& a, hipStream_t s) {
  constexpr size_t lds = bwd_sync_lds_bytes<NV>();
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_token_sync_kernel<E, NV, kC>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((bwd_token_sync_kernel<E, NV, kC>), dim3(static_cast<unsigned>((a.T + kSyncWavesB - 1) / kSyncWavesB)),
                     dim3(kSyncWavesB * kWave), lds, s, a);
  return hipGetLastError();
}
template <class E, int NV>
static hipError_t launch_bwd_sync(const BwdArgs& a, hipStream_t s) {
  if constexpr (E::kBytes == 2)
    if (a.C == 16) return launch_bwd_sync_c<E, NV, 16>(a, s);
  return launch_bwd_sync_c<E, NV, 0>(a, s);
}

// ---------------------------------------------------------------- row totals (for the split)
__global__ __launch_bounds__(256) void bwd_totals_kernel(BwdArgs p) {
  __shared__ int wtot[4];
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int n_t = p.F / p.tile_n;
  int total = 0;
  if (t < p.T) {
    for (int b = 0; b < n_t; ++b) total += max(p.count[t * n_t + b], 0);
    p.row_total[t] = total;
  }
  int st = total;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) st += __shfl_xor(st, o);
  if ((threadIdx.x & 63) == 0) wtot[threadIdx.x >> 6] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    p.block_total[blockIdx.x] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  }
}

// ---------------------------------------------------------------- per-neuron weight gradients
template <class E, int NV>
__global__ __launch_bounds__(4 * kWave, 2) void bwd_dw_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (j >= p.F) return;
  const int d = p.d;
  float ag[NV][kN], au[NV][kN], ad[NV][kN];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < kN; ++i) ag[v][i] = au[v][i] = ad[v][i] = 0.f;
  const int beg = p.neuron_off[j], end = p.neuron_off[j + 1];
  constexpr int kP = 2;
  for (int e0 = beg; e0 < end; e0 += kP) {
    float4 rr[kP];
    u32x4_t xv[kP][NV], yv[kP][NV];
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      const bool live = e0 + q < end;
      rr[q] = live ? p.recs[e0 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
      // clamped so that a corrupted record cannot address outside x / dy
      const int64_t t = min(max(static_cast<int64_t>(__float_as_int(rr[q].x)), int64_t(0)), p.T - 1);
      const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
      const u32x4_t* yr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.dy) + t * d * E::kBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        xv[q][v] = live ? xr[v * kWave + lane] : u32x4_t{0, 0, 0, 0};
        yv[q][v] = live ? yr[v * kWave + lane] : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int q = 0; q < kP; ++q) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float xf[kN], yf[kN];
        VecB<E>::unpack(xv[q][v], xf);
        VecB<E>::unpack(yv[q][v], yf);
#pragma unroll
        for (int i = 0; i < kN; ++i) {
          ag[v][i] = fmaf(rr[q].y, xf[i], ag[v][i]);
          au[v][i] = fmaf(rr[q].z, xf[i], au[v][i]);
          ad[v][i] = fmaf(rr[q].w, yf[i], ad[v][i]);
        }
      }
    }
  }
  float* og = p.dw_gate_t + j * d;
  float* ou = p.dw_up_t + j * d;
  float* od = p.dw_down + j * d;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t c = static_cast<int64_t>(v * kWave + lane) * kN;
#pragma unroll
    for (int i = 0; i < kN; i += 4) {
      *reinterpret_cast<f32x4_t*>(og + c + i) = f32x4_t{ag[v][i], ag[v][i + 1], ag[v][i + 2], ag[v][i + 3]};
      *reinterpret_cast<f32x4_t*>(ou + c + i) = f32x4_t{au[v][i], au[v][i + 1], au[v][i + 2], au[v][i + 3]};
      *reinterpret_cast<f32x4_t*>(od + c + i) = f32x4_t{ad[v][i], ad[v][i + 1], ad[v][i + 2], ad[v][i + 3]};
    }
  }
}

// ---------------------------------------------------------------- launch
template <class E, int NV>
static hipError_t launch_bwd_sparse_t(const BwdArgs& a, hipStream_t s) {
  // T == 0: no rows, so only the (all-zero) weight gradients are written
  const unsigned nblk = static_cast<unsigned>((a.T + kBlkRows - 1) / kBlkRows);
  const unsigned nchunk = static_cast<unsigned>((a.F + kNeuronChunk - 1) / kNeuronChunk);
  hipError_t e;
  if (nblk) {
    hipLaunchKernelGGL(bwd_hist_kernel, dim3(nblk, nchunk), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_colscan_kernel, dim3((a.F + 255) / 256), dim3(256), 0, s, a, static_cast<int>(nblk));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_nscan_kernel, dim3(1), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nblk) {
    hipLaunchKernelGGL(bwd_pos_kernel, dim3(nblk, nchunk), dim3(64), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (NV <= 4) {
      // light rows in lockstep, heavy rows cut into tile ranges
      const unsigned tblk = static_cast<unsigned>((a.T + 255) / 256);
      hipLaunchKernelGGL(bwd_totals_kernel, dim3(tblk), dim3(256), 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      RouteArgs r{};
      r.T = a.T;
      r.C = a.C;
      r.ell_rows = const_cast<int32_t*>(a.ell_rows);
      r.n_rows = const_cast<int32_t*>(a.n_rows);
      r.row_total = a.row_total;
      r.block_total = a.block_total;
      r.light_rows = a.light_rows;
      r.heavy_rows = a.heavy_rows;
      r.split_n = a.split_n;
      r.block_heavy = a.block_heavy;
      r.heavy_cap = a.heavy_cap;
      if ((e = launch_route_split(r, s)) != hipSuccess) return e;
      if ((e = launch_bwd_sync<E, NV>(a, s)) != hipSuccess) return e;
      const int64_t units = a.heavy_cap * a.groups;
      if (units > 0) {
        hipLaunchKernelGGL((bwd_token_kernel<E, NV, true>),
                           dim3(static_cast<unsigned>((units + kTokWaves - 1) / kTokWaves)), dim3(kTokWaves * kWave),
                           0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = launch_splitk_reduce(a.dx_hpart, a.groups, a.heavy_cap, a.split_n + 1, a.heavy_rows, a.dx, a.d,
                                 E::kBytes == 2 ? 1 : 0, s);
        if (e != hipSuccess) return e;
      }
    } else {
      hipLaunchKernelGGL((bwd_token_kernel<E, NV, false>),
                         dim3(static_cast<unsigned>((a.T + kTokWaves - 1) / kTokWaves)), dim3(kTokWaves * kWave), 0,
                         s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((bwd_dw_kernel<E, NV>), dim3(static_cast<unsigned>((a.F + 3) / 4)), dim3(4 * kWave), 0, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_bwd_sparse_e(const BwdArgs& a, hipStream_t s) {
  switch (a.d / (kWave * VecB<E>::N)) {
    case 1: return launch_bwd_sparse_t<E, 1>(a, s);
    case 2: return launch_bwd_sparse_t<E, 2>(a, s);
    case 3: return launch_bwd_sparse_t<E, 3>(a, s);
    case 4: return launch_bwd_sparse_t<E, 4>(a, s);
    case 5: return launch_bwd_sparse_t<E, 5>(a, s);
    case 6: return launch_bwd_sparse_t<E, 6>(a, s);
    case 7: return launch_bwd_sparse_t<E, 7>(a, s);
    case 8: return launch_bwd_sparse_t<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_sparse(const BwdArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_bwd_sparse_e<EBf16>(a, s) : launch_bwd_sparse_e<EF32>(a, s);
}

}  // namespace twell
