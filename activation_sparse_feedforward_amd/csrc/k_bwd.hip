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
//   mask     per block of 64 ELL rows and neuron, the 64-bit mask of the rows
//            holding it (within one row every neuron occurs at most once) and
//            its popcount
//   colscan  per neuron, exclusive scan of the counts over the blocks
//   nscan    exclusive scan over neurons -> start of each neuron's pair list
//   pos      per (row, tile), independent: a pair's place in its neuron's list
//            from the scans and a popcount of the mask below its row -> the
//            pair list {t, slot} in neuron-major order
//   dw       one wave per neuron j: W_up^T[j] and W_down[j] stay in VGPRs
//            while the wave walks j's pairs in ascending t, gathering x[t] and
//            dy[t]; it forms u, dh, dg, du, h for each pair, stores (dg, du)
//            in the pair's TwELL slot and keeps the three fp32 weight-gradient
//            rows in VGPRs; at the end it adds the dense rows' part (stored by
//            the dense-row GEMM, which runs first) and writes each row once
//   totals   per row, the sum of its counts; the ELL rows are then split into
//            light rows and at most heavy_cap heavy ones (row total >
//            max(2 C, 2 x mean)), as in the hybrid forward
//   dx       token-major: dx[t] = sum over t's slots of dg W_gate^T[j] +
//            du W_up^T[j], with (dg, du) read back from the slot.  Light rows:
//            16-wave workgroups walking the tiles in lockstep, so the weight
//            rows of the current tiles are shared through L2; heavy rows: one
//            wave per (row, tile range) with fp32 partial dx reduced in a
//            fixed order.
// Per pair each pass gathers two rows (x[t] and dy[t], then W_gate^T[j] and
// W_up^T[j]), and both dot products sit in the per-neuron pass, where one of
// their operands is already in registers.
#include "balance.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace twell {

namespace {

constexpr int kBlkRows = 64;         // ELL rows per counting-sort block
constexpr int kNeuronChunk = 2048;   // neurons per LDS mask table (16 KB); a multiple of every tile width
constexpr int kTokWaves = 4;
constexpr int kTokListCap = 512;

__device__ __forceinline__ int64_t n_ell_of(const BwdArgs& p) { return static_cast<int64_t>(p.n_rows[0]); }

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
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

}  // namespace

// ---------------------------------------------------------------- row masks
// Per block of 64 ELL rows and neuron j: a 64-bit mask of the block's rows
// whose stored slots hold j (bit r = row 64 blk + r); its popcount is the
// block's count for j.
__global__ __launch_bounds__(256) void bwd_mask_kernel(BwdArgs p) {
  __shared__ unsigned long long mask[kNeuronChunk];
  __shared__ int64_t rows[kBlkRows];
  const int blk = blockIdx.x;
  const int j0 = blockIdx.y * kNeuronChunk;
  const int nj = min(kNeuronChunk, p.F - j0);
  for (int j = threadIdx.x; j < nj; j += 256) mask[j] = 0ull;
  const int64_t n_ell = n_ell_of(p);
  const int64_t i0 = static_cast<int64_t>(blk) * kBlkRows;
  if (threadIdx.x < kBlkRows) rows[threadIdx.x] = i0 + threadIdx.x < n_ell ? p.ell_rows[i0 + threadIdx.x] : -1;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_t = p.F / p.tile_n;
  // only this chunk's tiles; a wave's 16 rows x those tiles are spread over its
  // lanes, so each lane walks a few (row, tile) items instead of 16 rows
  const int b0 = j0 / p.tile_n, nb = nj / p.tile_n;
  constexpr int kRowsPerWave = kBlkRows / 4;
  for (int it = lane; it < kRowsPerWave * nb; it += 64) {
    const int r = wave * kRowsPerWave + it / nb;
    const int b = b0 + it % nb;
    const int64_t t = rows[r];
    if (t < 0) continue;
    const int cnt = max(0, min(p.count[t * n_t + b], p.C));
    const int64_t rec = (t * n_t + b) * p.C;
    for (int s = 0; s < cnt; ++s) {
      const int j = b * p.tile_n + (p.idx[rec + s] & (p.tile_n - 1)) - j0;
      if (j >= 0 && j < nj) atomicOr(&mask[j], 1ull << r);
    }
  }
  __syncthreads();
  const int64_t o = static_cast<int64_t>(blk) * p.F + j0;
  for (int j = threadIdx.x; j < nj; j += 256) {
    const unsigned long long m = mask[j];
    p.blk_mask[o + j] = m;
    p.blk_hist[o + j] = __popcll(m);
  }
}

// ---------------------------------------------------------------- column scan
// Per neuron, exclusive scan of the block counts over the blocks (in place);
// the total goes to neuron_off[j].  A workgroup takes 32 neurons, each in 8
// segments of blocks summed in parallel.
__global__ __launch_bounds__(256) void bwd_colscan_kernel(BwdArgs p, int nblk) {
  __shared__ int seg_sum[8][32];
  const int jl = threadIdx.x & 31, seg = threadIdx.x >> 5;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 32 + jl;
  const int per = (nblk + 7) / 8;
  const int b0 = min(nblk, seg * per), b1 = min(nblk, b0 + per);
  int32_t* h = p.blk_hist + j;
  int sum = 0;
  if (j < p.F)
    for (int b = b0; b < b1; ++b) sum += h[static_cast<int64_t>(b) * p.F];
  seg_sum[seg][jl] = sum;
  __syncthreads();
  int run = 0;
  for (int k = 0; k < seg; ++k) run += seg_sum[k][jl];
  if (j < p.F) {
    for (int b = b0; b < b1; ++b) {
      const int c = h[static_cast<int64_t>(b) * p.F];
      h[static_cast<int64_t>(b) * p.F] = run;
      run += c;
    }
    if (seg == 7) p.neuron_off[j] = run;  // per-neuron total; turned into offsets by nscan
  }
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
    const int incl = wave_incl_scan(v);
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

// ---------------------------------------------------------------- positions
// One thread per (ELL row i, tile): the pair (i, j) goes to
//   neuron_off[j] + (pairs of j in earlier blocks) + (rows of i's block
//   before i that hold j),
// the last term a popcount of the block's row mask below bit i % 64, so each
// neuron's pairs come out in ascending i (= ascending t) with no ordering
// between threads.
__global__ __launch_bounds__(256) void bwd_pos_kernel(BwdArgs p) {
  const int n_t = p.F / p.tile_n;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t i = u / n_t;
  const int b = static_cast<int>(u - i * n_t);
  if (i >= n_ell_of(p)) return;
  const int64_t t = p.ell_rows[i];
  const int cnt = max(0, min(p.count[t * n_t + b], p.C));
  const int r = static_cast<int>(i & (kBlkRows - 1));
  const unsigned long long below = (1ull << r) - 1ull;
  const int64_t blk_off = (i / kBlkRows) * p.F;
  const int64_t rec = (t * n_t + b) * p.C;
  for (int s = 0; s < cnt; ++s) {
    const int j = b * p.tile_n + (p.idx[rec + s] & (p.tile_n - 1));
    const int q = p.neuron_off[j] + p.blk_hist[blk_off + j] + __popcll(p.blk_mask[blk_off + j] & below);
    p.pairs[q] = make_int2(static_cast<int>(t), static_cast<int>(rec + s));
  }
}

// ---------------------------------------------------------------- per-neuron pass
// One wave per neuron j.  Its W_up^T and W_down rows are loaded once and stay
// in VGPRs; for each pair (t, slot) in ascending t the wave gathers x[t] and
// dy[t] and forms
//     u = x[t].W_up^T[j], e = dy[t].W_down[j], h = a u, dh = e + l1 sign(h),
//     du = dh a, dg = dh u
// (a = the slot's stored ReLU value).  (dg, du) go to the slot for the dx
// pass; dg x[t], du x[t] and h dy[t] accumulate into fp32 rows in VGPRs.
// Two waves share a SIMD, with two pairs in flight per iteration up to 4
// 16-byte vectors per lane and one above; rows too wide for that (bf16
// d_model >= 3072: three fp32 rows, the two weight rows and a pair's x and dy
// pass 230 VGPRs) give the wave the SIMD to itself with two pairs in flight:
// the same pairs in flight per CU, no spills.
template <class E, int NV>
struct DwShape {
  static constexpr int kOnePair = NV * (3 * VecB<E>::N + 16);  // VGPRs per lane, one pair in flight
  static constexpr bool kWide = kOnePair > 230;
  static constexpr int kWavesPerSimd = kWide ? 1 : 2;
  static constexpr int kPairs = (NV <= 4 || kWide) ? 2 : 1;
};

template <class E, int NV>
__global__ __launch_bounds__(4 * kWave, (DwShape<E, NV>::kWavesPerSimd)) void bwd_dw_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (j >= p.F) return;
  const int d = p.d;
  u32x4_t wu[NV], wd[NV];
  {
    const int64_t ro = j * d * E::kBytes;
    const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
    const u32x4_t* dr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + ro);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      // the neuron's own rows are read by this wave only
      wu[v] = __builtin_nontemporal_load(ur + v * kWave + lane);
      wd[v] = __builtin_nontemporal_load(dr + v * kWave + lane);
    }
  }
  float ag[NV][kN], au[NV][kN], ad[NV][kN];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < kN; ++i) ag[v][i] = au[v][i] = ad[v][i] = 0.f;
  const int beg = p.neuron_off[j], end = p.neuron_off[j + 1];
  constexpr int kP = DwShape<E, NV>::kPairs;
  for (int e0 = beg; e0 < end; e0 += kP) {
    float aq[kP];
    int sq[kP];
    u32x4_t xv[kP][NV], yv[kP][NV];
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      const bool live = e0 + q < end;
      const int2 pr = live ? p.pairs[e0 + q] : make_int2(0, 0);
      sq[q] = pr.y;
      aq[q] = live ? load_elem<E>(p.val, pr.y) : 0.f;
      // clamped so that a corrupted pair cannot address outside x / dy
      const int64_t t = min(max(static_cast<int64_t>(pr.x), int64_t(0)), p.T - 1);
      const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
      const u32x4_t* yr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.dy) + t * d * E::kBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        xv[q][v] = live ? xr[v * kWave + lane] : u32x4_t{0, 0, 0, 0};
        yv[q][v] = live ? yr[v * kWave + lane] : u32x4_t{0, 0, 0, 0};
      }
    }
    float uq[kP], eq[kP];
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      uq[q] = row_dot<E, NV>(wu, xv[q]);
      eq[q] = row_dot<E, NV>(wd, yv[q]);
    }
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      uq[q] = wave_sum(uq[q]);
      eq[q] = wave_sum(eq[q]);
    }
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      // a dead pair has a = 0 and zero rows, so it adds nothing
      const float a = aq[q], u = uq[q];
      const float h = a * u;
      const float sg = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
      const float dh = eq[q] + p.l1 * sg;
      const float du = dh * a;
      const float dg = dh * u;
      if (e0 + q < end && lane == 0) p.coef[sq[q]] = make_float2(dg, du);
      const AxpyCoef<E> cg(dg), cu(du), ch(h);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        cg.axpy(xv[q][v], ag[v]);
        cu.axpy(xv[q][v], au[v]);
        ch.axpy(yv[q][v], ad[v]);
      }
    }
  }
  float* og = p.dw_gate_t + j * d;
  float* ou = p.dw_up_t + j * d;
  float* od = p.dw_down + j * d;
  // the dense rows' GEMM ran first and stored their part of these rows: added
  // here, once (with no dense rows it wrote nothing, and an empty batch has cap 0
  // so n_rows is not read)
  const bool from_dense = p.cap > 0 && p.n_rows[1] > 0;  // uniform
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int64_t c = static_cast<int64_t>(v * kWave + lane) * kN;
#pragma unroll
    for (int i = 0; i < kN; i += 4) {
      f32x4_t rg = f32x4_t{ag[v][i], ag[v][i + 1], ag[v][i + 2], ag[v][i + 3]};
      f32x4_t ru = f32x4_t{au[v][i], au[v][i + 1], au[v][i + 2], au[v][i + 3]};
      f32x4_t rd = f32x4_t{ad[v][i], ad[v][i + 1], ad[v][i + 2], ad[v][i + 3]};
      if (from_dense) {
        rg += *reinterpret_cast<const f32x4_t*>(og + c + i);
        ru += *reinterpret_cast<const f32x4_t*>(ou + c + i);
        rd += *reinterpret_cast<const f32x4_t*>(od + c + i);
      }
      *reinterpret_cast<f32x4_t*>(og + c + i) = rg;
      *reinterpret_cast<f32x4_t*>(ou + c + i) = ru;
      *reinterpret_cast<f32x4_t*>(od + c + i) = rd;
    }
  }
}

// ---------------------------------------------------------------- dx pass
// dx[t] = sum over t's stored slots of dg W_gate^T[j] + du W_up^T[j], with
// (dg, du) written to the slot by the per-neuron pass.  The tiles are walked in
// ascending order, so every row's sum has a fixed order.

// One wave per ELL row (SPLIT = false: every ELL row; used where the lockstep
// kernel does not fit), or per (heavy row, tile range) with fp32 partial dx
// written to dx_hpart[range][i][:] (SPLIT = true).
template <class E, int NV, bool SPLIT>
__global__ __launch_bounds__(kTokWaves * kWave, 2) void bwd_ell_dx_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  constexpr int kU = NV <= 2 ? 4 : 2;
  __shared__ int2 list_all[kTokWaves][kTokListCap];
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
  int2* list = list_all[wave];
  float dxf[NV][kN];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < kN; ++i) dxf[v][i] = 0.f;
  const int chunk_tiles = min(kWave, kTokListCap / C);
  for (int b0 = b_begin; b0 < b_end; b0 += chunk_tiles) {
    const int b = b0 + lane;
    int cnt = 0;
    if (lane < chunk_tiles && b < b_end) cnt = max(0, min(p.count[t * n_t + b], C));
    const int incl = wave_incl_scan(cnt);
    const int total = wave_last(incl);
    const int off = incl - cnt;
    if (cnt > 0) {
      const int64_t rec = (t * n_t + b) * C;
      for (int s = 0; s < cnt; ++s)
        list[off + s] = make_int2(b * tile_n + (p.idx[rec + s] & (tile_n - 1)), static_cast<int>(rec + s));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e0 = 0; e0 < total; e0 += kU) {
      const int nq = min(kU, total - e0);
      int jj[kU];
      float2 cf[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int2 ent = list[min(e0 + q, total - 1)];
        jj[q] = __builtin_amdgcn_readfirstlane(ent.x);
        cf[q] = q < nq ? p.coef[__builtin_amdgcn_readfirstlane(ent.y)] : make_float2(0.f, 0.f);
      }
      u32x4_t wg[kU][NV], wu[kU][NV];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int64_t ro = int64_t(jj[q]) * d * E::kBytes;
        const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_gate_t) + ro);
        const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
        if (q < nq) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            wg[q][v] = gr[v * kWave + lane];
            wu[q][v] = ur[v * kWave + lane];
          }
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) wg[q][v] = wu[q][v] = u32x4_t{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const AxpyCoef<E> cg(cf[q].x), cu(cf[q].y);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          cu.axpy(wu[q][v], dxf[v]);
          cg.axpy(wg[q][v], dxf[v]);
        }
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

// Light rows in lockstep: kW waves of TPW rows each, fp32 dx rows in VGPRs
// (16 waves up to bf16 d_model = 2048; 8 above, whose two rows per wave need
// the 256 VGPRs of two waves per SIMD).  Every chunk of tiles starts with a
// workgroup barrier, so the resident workgroups sweep the neurons in roughly
// the same order and the two weight rows of each pair are reused from L2;
// each XCD's workgroups (dealt round-robin) start at a different chunk and
// wrap around.
constexpr int kDxWaves = 16;
constexpr int kDxWavesWide = 8;
constexpr int64_t kDxWideBatch = 4096;  // rows from which wider rows take the lockstep dx pass
constexpr int kDxList = 128;      // {j, slot, row} entries per wave per chunk
constexpr int kDxChunkMax = 4;
// a chunk's weight rows at most one XCD's L2: 4 tiles x 128 neurons x 2 rows x
// 4 KB = 4 MB at d_model = 2048, 2 tiles at 4096
constexpr int64_t kDxChunkBytes = int64_t(4) << 20;

template <int kW>
constexpr size_t bwd_dx_sync_lds_bytes() { return static_cast<size_t>(kW) * kDxList * 16; }

template <class E, int NV, int TPW, int kC, int kW>
__global__ __launch_bounds__(kW * kWave) void bwd_ell_dx_sync_kernel(BwdArgs p) {
  constexpr int kN = VecB<E>::N;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int4* list = reinterpret_cast<int4*>(smem) + wave * kDxList;
  const int d = p.d, C = kC > 0 ? kC : p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  const int64_t n_rows = p.split_n[0];
  const int64_t blk = p.blk0 + blockIdx.x;  // row block of this workgroup
  // rows are dealt over windows of workgroups (balance_rows): only a workgroup
  // whose whole window is past the rows has none
  if (blk / kBalanceWindow * kBalanceWindow * kW * TPW >= n_rows) return;
  int64_t src[TPW];
  // the ranking's scratch sits in the entry lists, first written after the
  // barrier that opens the first chunk
  balance_rows<kW, TPW, kBalanceWindow>(p.count, p.row_total, p.light_rows, n_rows, n_t, blk,
                                        (p.T + kW * TPW - 1) / (kW * TPW), kBalanceWindow, wave,
                                        reinterpret_cast<int*>(smem), src);
  int64_t tk[TPW];
  bool act[TPW];
  float dxf[TPW][NV][kN];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int64_t i_row = src[k];
    act[k] = i_row < n_rows;  // idle rows: the wave still takes part in the barriers
    tk[k] = act[k] ? static_cast<int64_t>(__builtin_amdgcn_readfirstlane(p.light_rows[i_row])) : 0;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < kN; ++i) dxf[k][v][i] = 0.f;
  }
  // list builder lanes: lane = tile_in_chunk * TPW + row
  const int l2_tiles = static_cast<int>(kDxChunkBytes / (int64_t(tile_n) * 2 * d * E::kBytes));
  const int chunk_tiles = max(1, min(min(kWave / TPW, kDxList / (C * TPW)), min(kDxChunkMax, l2_tiles)));
  const int n_chunks = (n_t + chunk_tiles - 1) / chunk_tiles;
  // a later generation starts one chunk earlier than the one before it, on the
  // chunk its XCD's previous generation swept last (still in L2)
  const int gen_r = p.resident > 0 ? static_cast<int>(blk / p.resident) : 0;
  const int rot = ((static_cast<int>(blk & 7) * (n_chunks / 8) - gen_r) % n_chunks + n_chunks) % n_chunks;
  const int kl = lane % TPW;
  int my_tok = 0;  // token rows are < 2^31
  bool my_act = false;
#pragma unroll
  for (int k = 0; k < TPW; ++k)
    if (kl == k) {
      my_tok = static_cast<int>(tk[k]);
      my_act = act[k] && lane < chunk_tiles * TPW;
    }
  // C = 16: the builder lane's count and 16 index bytes of the next chunk are
  // loaded while the current chunk's entries are processed.
  int pf_cnt = 0;
  u32x4_t pf_idx{0, 0, 0, 0};
  auto prefetch = [&](int c) {
    const int b = ((c + rot) % n_chunks) * chunk_tiles + lane / TPW;
    pf_cnt = 0;
    if (my_act && b < n_t) {
      const int64_t rec = static_cast<int64_t>(my_tok) * n_t + b;
      pf_cnt = __builtin_nontemporal_load(p.count + rec);
      pf_idx = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p.idx + rec * 16));
    }
  };
  if constexpr (kC == 16) prefetch(0);
  for (int c = 0; c < n_chunks; ++c) {
    const int b0 = ((c + rot) % n_chunks) * chunk_tiles;
    __syncthreads();
    const int b = b0 + lane / TPW;
    int total;
    if constexpr (kC == 16) {
      const int cnt = max(0, min(pf_cnt, 16));
      const u32x4_t ix = pf_idx;
      const int spos = (my_tok * n_t + b) * 16;
      const int incl = wave_incl_scan(cnt);
      total = min(wave_last(incl), kDxList);
      const int off = incl - cnt;
      // slots up to the largest count of the builder lanes
      int n_s = 0;
      while (n_s < 16 && __builtin_amdgcn_ballot_w64(cnt > n_s)) ++n_s;
      for (int s2 = 0; s2 < n_s; ++s2) {
        if (s2 < cnt && off + s2 < kDxList) {
          const uint32_t w = s2 < 8 ? (s2 < 4 ? ix[0] : ix[1]) : (s2 < 12 ? ix[2] : ix[3]);
          const int j = b * tile_n + (static_cast<int>((w >> (8 * (s2 & 3))) & 0xffu) & (tile_n - 1));
          list[off + s2] = make_int4(j, spos + s2, kl, 0);
        }
      }
      if (c + 1 < n_chunks) prefetch(c + 1);
    } else {
      int cnt = 0;
      if (my_act && b < n_t) cnt = max(0, min(p.count[static_cast<int64_t>(my_tok) * n_t + b], C));
      const int incl = wave_incl_scan(cnt);
      total = min(wave_last(incl), kDxList);
      const int off = incl - cnt;
      if (cnt > 0) {
        const int rec = (my_tok * n_t + b) * C;
        // off + cnt <= chunk_tiles * TPW * C <= kDxList by the launch's choice of TPW
        for (int s2 = 0; s2 < cnt && off + s2 < kDxList; ++s2)
          list[off + s2] = make_int4(b * tile_n + (p.idx[rec + s2] & (tile_n - 1)), rec + s2, kl, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e = 0; e < total; ++e) {
      const int4 ent = list[e];
      const int j = __builtin_amdgcn_readfirstlane(ent.x);
      const float2 cf = p.coef[__builtin_amdgcn_readfirstlane(ent.y)];
      const int kk = __builtin_amdgcn_readfirstlane(ent.z);
      const int64_t ro = int64_t(j) * d * E::kBytes;
      const u32x4_t* gr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_gate_t) + ro);
      const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
      u32x4_t wg[NV], wu[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        wg[v] = gr[v * kWave + lane];
        wu[v] = ur[v * kWave + lane];
      }
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        if (kk == k) {  // wave-uniform
          const AxpyCoef<E> cg(cf.x), cu(cf.y);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            cu.axpy(wu[v], dxf[k][v]);
            cg.axpy(wg[v], dxf[k][v]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    if (act[k]) {
      u32x4_t* dxr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dx) + tk[k] * d * E::kBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(VecB<E>::pack(dxf[k][v]), dxr + v * kWave + lane);
    }
  }
}

template <class E, int NV, int TPW, int kC, int kW>
static hipError_t launch_bwd_dx_sync_c(const BwdArgs& args, hipStream_t s) {
  BwdArgs a = args;
  a.resident = lockstep_resident();
  constexpr size_t lds = bwd_dx_sync_lds_bytes<kW>();
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_ell_dx_sync_kernel<E, NV, TPW, kC, kW>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  constexpr int64_t per_block = static_cast<int64_t>(kW) * TPW;
  const int64_t blocks = (a.T + per_block - 1) / per_block;
  // one launch per generation of resident workgroups (as the forward's lockstep kernel)
  const int64_t step = a.resident > 0 ? a.resident : blocks;
  for (int64_t b0 = 0; b0 < blocks; b0 += step) {
    a.blk0 = b0;
    hipLaunchKernelGGL((bwd_ell_dx_sync_kernel<E, NV, TPW, kC, kW>),
                       dim3(static_cast<unsigned>(blocks - b0 < step ? blocks - b0 : step)), dim3(kW * kWave), lds, s,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
// Rows per wave: two fp32 dx rows beside one pair's two weight rows fit the
// 128 VGPRs of a 16-wave workgroup up to d_model = 2048 (bf16) / 1024 (fp32),
// and the 256 of an 8-wave workgroup up to bf16 d_model = 4096; TPW * C <=
// kDxList, so every chunk of >= 1 tile fits the list.
template <class E, int NV>
static hipError_t launch_bwd_dx_sync(const BwdArgs& a, hipStream_t s) {
  constexpr int kW = NV * VecB<E>::N <= 32 ? kDxWaves : kDxWavesWide;
  constexpr bool two = NV * VecB<E>::N <= 32 || kW == kDxWavesWide;
  if constexpr (E::kBytes == 2)
    if (a.C == 16) return launch_bwd_dx_sync_c<E, NV, two ? 2 : 1, 16, kW>(a, s);
  if (two && 2 * a.C <= kDxList) return launch_bwd_dx_sync_c<E, NV, two ? 2 : 1, 0, kW>(a, s);
  return launch_bwd_dx_sync_c<E, NV, 1, 0, kW>(a, s);
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

// ---------------------------------------------------------------- launch
template <class E, int NV>
static hipError_t launch_bwd_sparse_t(const BwdArgs& a, hipStream_t s) {
  // T == 0: no rows, so only the (all-zero) weight gradients are written
  const unsigned nblk = static_cast<unsigned>((a.T + kBlkRows - 1) / kBlkRows);
  const unsigned nchunk = static_cast<unsigned>((a.F + kNeuronChunk - 1) / kNeuronChunk);
  hipError_t e;
  if (nblk) {
    hipLaunchKernelGGL(bwd_mask_kernel, dim3(nblk, nchunk), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_colscan_kernel, dim3((a.F + 31) / 32), dim3(256), 0, s, a, static_cast<int>(nblk));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_nscan_kernel, dim3(1), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nblk) {
    const int64_t units = a.T * (a.F / a.tile_n);  // (row, tile) pairs; rows past n_ell exit
    hipLaunchKernelGGL(bwd_pos_kernel, dim3(static_cast<unsigned>((units + 255) / 256)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // per-neuron pass: the weight gradients (zero rows when T == 0) and the
  // (dg, du) of every stored slot, which the dx pass reads
  hipLaunchKernelGGL((bwd_dw_kernel<E, NV>), dim3(static_cast<unsigned>((a.F + 3) / 4)), dim3(4 * kWave), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!nblk) return hipSuccess;
  // light rows in lockstep, heavy rows cut into tile ranges; bf16 rows wider
  // than 2048 only from kDxWideBatch rows on (below, the 8-wave lockstep
  // workgroups leave most CUs idle), fp32 rows wider than 1024 never
  if constexpr (NV <= 4 || E::kBytes == 2) {
    if (NV <= 4 || a.T >= kDxWideBatch) {
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
      if ((e = launch_bwd_dx_sync<E, NV>(a, s)) != hipSuccess) return e;
      const int64_t units = a.heavy_cap * a.groups;
      if (units > 0) {
        hipLaunchKernelGGL((bwd_ell_dx_kernel<E, NV, true>),
                           dim3(static_cast<unsigned>((units + kTokWaves - 1) / kTokWaves)), dim3(kTokWaves * kWave), 0,
                           s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = launch_splitk_reduce(a.dx_hpart, a.groups, a.heavy_cap, a.split_n + 1, a.heavy_rows, a.dx, a.d,
                                 E::kBytes == 2 ? 1 : 0, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  hipLaunchKernelGGL((bwd_ell_dx_kernel<E, NV, false>), dim3(static_cast<unsigned>((a.T + kTokWaves - 1) / kTokWaves)),
                     dim3(kTokWaves * kWave), 0, s, a);
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
