// Fused TwELL up + down projection: one fused kernel (the lockstep variant is
// dispatched once per generation of resident workgroups, on disjoint rows).
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
#include "balance.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace twell {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kListCap = 1024;  // list entries per wave and per chunk of tiles

// Neurons in flight per wave: enough 16-byte loads outstanding to cover the
// gather latency, without spilling at the widest rows.
template <int NV> constexpr int neurons_in_flight() { return NV <= 1 ? 8 : (NV <= 4 ? 4 : 2); }


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

// This lane's part of the dot product of two rows held as NV 16-byte chunks
// (x and w in storage form).  bf16: packed-pair dot products (v_dot2 with an
// fp32 accumulator) in four independent chains, summed at the end; fp32:
// plain FMAs in the same four-chain order.  (The bf16 pairs are taken from a
// whole-vector cast: casting an element of the 32-bit vector directly was
// compiled to always read element 0.)
template <class E, int NV>
__device__ __forceinline__ float lane_dot(const u32x4_t* w, const u32x4_t* x) {
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

// One 16-byte piece of lane_dot, accumulated into the same four chains.
template <class E>
__device__ __forceinline__ void lane_dot_piece(const u32x4_t& w, const u32x4_t& x, float (&acc)[4]) {
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

// NV = 16-byte vectors per lane per row: d_model = NV * 64 * Vec<E>::N.
// SPLIT: each row of the list is cut into p.groups tile ranges, one wave per
// (row, range), writing its fp32 partial y to p.part[range][i_row][:] for a
// fixed-order reduction afterwards (used for the few rows with far more
// non-zeros than the rest, which would otherwise serialise on one wave).
template <class E, int NV, bool SPLIT>
__global__ __launch_bounds__(kWavesPerBlock * kWave, 2) void fused_updown_kernel(FusedArgs p) {
  constexpr int kN = Vec<E>::N;
  constexpr int kU = neurons_in_flight<NV>();
  __shared__ int2 list_all[kWavesPerBlock][kListCap];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.T;
  const int d = p.d, C = p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  int64_t i_row = unit;
  int grp = 0, b_begin = 0, b_end = n_t;
  if constexpr (SPLIT) {
    n_rows = min(n_rows, p.part_rows);
    if (unit >= n_rows * p.groups) return;
    i_row = unit / p.groups;
    grp = static_cast<int>(unit - i_row * p.groups);
    const int tg = (n_t + p.groups - 1) / p.groups;
    b_begin = min(n_t, grp * tg);
    b_end = min(n_t, b_begin + tg);
  } else {
    if (i_row >= n_rows) return;  // whole wave exits together; no block barrier below
  }
  const int64_t t = p.rows ? static_cast<int64_t>(p.rows[i_row]) : i_row;
  int2* list = list_all[wave];

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
  for (int b0 = b_begin; b0 < b_end; b0 += chunk_tiles) {
    // ---- build the (j, a) list of this chunk of tiles, ascending j
    const int b = b0 + lane;
    int cnt = 0;
    // counts are clamped to [0, C] and tile-local indices masked to the tile
    // width (a power of two), so even a corrupted TwELL stays in bounds
    if (lane < chunk_tiles && b < b_end) cnt = max(0, min(p.count[t * n_t + b], C));
    const int incl = wave_incl_scan(cnt);
    const int total = wave_last(incl);
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
      for (int q = 0; q < kU; ++q) hq[q] = lane_dot<E, NV>(wu[q], xs);
#pragma unroll
      for (int q = 0; q < kU; ++q) hq[q] = aa[q] * wave_sum(hq[q]);
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const AxpyCoef<E> hc(hq[q]);
#pragma unroll
        for (int v = 0; v < NV; ++v) hc.axpy(wd[q][v], yf[v]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  if constexpr (SPLIT) {
    float* o = p.part + (static_cast<int64_t>(grp) * p.part_rows + i_row) * d;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < kN; i += 4)
        *reinterpret_cast<float4*>(o + (v * kWave + lane) * kN + i) =
            make_float4(yf[v][i], yf[v][i + 1], yf[v][i + 2], yf[v][i + 3]);
  } else {
    u32x4_t* yr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.y) + t * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) yr[v * kWave + lane] = Vec<E>::pack(yf[v]);
  }
}

// Lockstep variant (d_model up to 2048 in bf16): a workgroup of 16 waves, each
// owning TPW tokens, walks the TwELL tiles in chunks with a workgroup barrier
// between chunks (while a chunk's rows fill an XCD's L2; narrower rows run
// free, see chunk_sync).  Every resident workgroup therefore sweeps the neuron tiles
// in roughly the same order at the same time, so the weight rows of the
// current tiles (~1 MB per tile at the 2B shape) are shared through each
// XCD's L2 instead of each wave fetching random rows from the MALL; more
// tokens per workgroup keeps the workgroups in tighter step.  x[t] lives in
// LDS (this frees the VGPRs for the fp32 y accumulators of TPW tokens).  Per
// token the arithmetic is that of fused_updown_kernel, with the tiles summed
// starting from the workgroup's rotated chunk (a function of the workgroup
// index, so results are deterministic for a given row list).  Rows are dealt
// to the waves by their entry counts (balance_rows: within each workgroup for
// all rows, over windows of 8 workgroups for a row list), which shortens the
// wait at every chunk barrier and keeps the workgroups in step.  Workgroups
// have 16 waves up to 4 16-byte vectors per lane (bf16 d_model <= 2048) and 8
// above (bf16 d_model <= 4096), where two fp32 y rows per wave need the 256
// VGPRs of two waves per SIMD.
constexpr int kSyncWaves = 16;
constexpr int kSyncWavesWide = 8;
constexpr int kSyncList = 128;  // list entries per wave per chunk
constexpr int kSyncChunkMax = 4;
// a chunk's weight rows (tiles x T_n neurons x 2 rows) are at most one XCD's L2
constexpr int64_t kSyncChunkBytes = int64_t(4) << 20;

template <class E, int NV, int TPW, int kU, int kC, int kW>
__global__ __launch_bounds__(kW * kWave) void fused_updown_sync_kernel(FusedArgs p) {
  constexpr int kN = Vec<E>::N;
  constexpr int kRowVec = NV * kWave;  // 16-byte vectors per row
  extern __shared__ __align__(16) char smem[];
  u32x4_t* xl = reinterpret_cast<u32x4_t*>(smem);  // [16 waves][TPW][kRowVec]
  int4* list_all = reinterpret_cast<int4*>(smem + kW * TPW * kRowVec * 16);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.T;
  const int64_t blk = p.blk0 + blockIdx.x;  // row block of this workgroup
  // rows are dealt over windows of workgroups (balance_rows): only a workgroup
  // whose whole window is past the rows has none
  const int win = p.rows ? kBalanceWindow : 1;
  if (blk / win * win * kW * TPW >= n_rows) return;
  int4* list = list_all + wave * kSyncList;
  u32x4_t* xw = xl + wave * TPW * kRowVec;
  const int d = p.d, C = kC > 0 ? kC : p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  int64_t src[TPW];
  // the ranking's scratch sits in the entry lists, first written after the
  // barrier that opens the first chunk
  balance_rows<kW, TPW, kBalanceWindow>(p.count, p.row_total, p.rows, n_rows, n_t, blk,
                                        (p.T + kW * TPW - 1) / (kW * TPW), win, wave,
                                                reinterpret_cast<int*>(list_all), src);

  int64_t tk[TPW];
  bool act[TPW];
  float yf[TPW][NV][kN];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int64_t i_row = src[k];
    act[k] = i_row < n_rows;  // idle tokens: the wave still takes part in the barriers
    // wave-uniform: keep the token rows in scalar registers
    tk[k] = act[k] ? (p.rows ? static_cast<int64_t>(__builtin_amdgcn_readfirstlane(p.rows[i_row])) : i_row) : 0;
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + tk[k] * d * E::kBytes);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      // x, the counts / indices and y are touched once: non-temporal accesses
      // keep them from pushing the shared weight rows out of L2
      xw[k * kRowVec + v * kWave + lane] =
          act[k] ? __builtin_nontemporal_load(xr + v * kWave + lane) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kN; ++i) yf[k][v][i] = 0.f;
    }
  }
  // lanes of the list builder: lane = tile_in_chunk * TPW + token
  // at most 4 tiles per chunk, and no more than an XCD's L2 holds of their
  // weight rows (4 x 128 neurons x 2 rows x d_model x 2 B = 4 MB at d_model =
  // 2048; 2 tiles at 4096)
  const int l2_tiles = static_cast<int>(kSyncChunkBytes / (int64_t(tile_n) * 2 * d * E::kBytes));
  const int chunk_tiles = max(1, min(min(kWave / TPW, kSyncList / (C * TPW)), min(kSyncChunkMax, l2_tiles)));
  // Workgroups are dealt round-robin to the 8 XCDs; each XCD's workgroups start
  // their sweep at a different chunk (and wrap around), so the XCDs do not all
  // request the same weight rows from the MALL at the same time.
  const int n_chunks = (n_t + chunk_tiles - 1) / chunk_tiles;
  // The barrier at each chunk keeps the workgroup's waves on the chunk's rows
  // while those rows fill an XCD's L2.  When they take half of it or less
  // (rows of 2 KB and narrower, e.g. bf16 d_model = 1024), the waves run free
  // after the first chunk: the rows of the chunks the waves drift over still
  // fit, and the waits at the barriers cost more than they save.  The first
  // barrier stays: it orders the ranking's scratch before the first lists.
  // The summation order does not depend on it.
  const bool chunk_sync = int64_t(chunk_tiles) * tile_n * 2 * d * E::kBytes * 2 > kSyncChunkBytes;
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
  // loaded while the current chunk's entries are processed, so a chunk starts
  // without waiting on global memory; an entry carries the position of its
  // value, which is loaded beside the entry's weight rows.
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
    if (c == 0 || chunk_sync) __syncthreads();
    const int b = b0 + lane / TPW;
    int total;
    if constexpr (kC == 16) {
      const int cnt = max(0, min(pf_cnt, 16));
      const u32x4_t ix = pf_idx;
      const int vpos = (my_tok * n_t + b) * 16;
      const int incl = wave_incl_scan(cnt);
      total = min(wave_last(incl), kSyncList);
      const int off = incl - cnt;
      // slots up to the largest count of the builder lanes (a builder lane
      // rarely holds more than a few entries of a chunk)
      int n_s = 0;
      while (n_s < 16 && __builtin_amdgcn_ballot_w64(cnt > n_s)) ++n_s;
      for (int s2 = 0; s2 < n_s; ++s2) {
        if (s2 < cnt && off + s2 < kSyncList) {
          const uint32_t w = s2 < 8 ? (s2 < 4 ? ix[0] : ix[1]) : (s2 < 12 ? ix[2] : ix[3]);
          const int j = b * tile_n + (static_cast<int>((w >> (8 * (s2 & 3))) & 0xffu) & (tile_n - 1));
          list[off + s2] = make_int4(j, vpos + s2, kl, 0);
        }
      }
      if (c + 1 < n_chunks) prefetch(c + 1);
    } else {
      int cnt = 0;
      if (my_act && b < n_t) cnt = max(0, min(p.count[static_cast<int64_t>(my_tok) * n_t + b], C));
      const int incl = wave_incl_scan(cnt);
      total = min(wave_last(incl), kSyncList);
      const int off = incl - cnt;
      if (cnt > 0) {
        const int64_t rec = (static_cast<int64_t>(my_tok) * n_t + b) * C;
        // off + cnt <= chunk_tiles * TPW * C <= kSyncList by the launch's choice of TPW
        for (int s2 = 0; s2 < cnt && off + s2 < kSyncList; ++s2) {
          const int j = b * tile_n + (p.idx[rec + s2] & (tile_n - 1));
          list[off + s2] = make_int4(j, __float_as_int(load_elem<E>(p.val, rec + s2)), kl, 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e0 = 0; e0 < total; e0 += kU) {
      const int nq = min(kU, total - e0);
      int jj[kU], kk[kU];
      float aa[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int4 ent = list[min(e0 + q, total - 1)];
        jj[q] = __builtin_amdgcn_readfirstlane(ent.x);
        if constexpr (kC == 16)
          aa[q] = (q < nq) ? load_elem<E>(p.val, __builtin_amdgcn_readfirstlane(ent.y)) : 0.f;
        else
          aa[q] = (q < nq) ? __int_as_float(__builtin_amdgcn_readfirstlane(ent.y)) : 0.f;
        kk[q] = __builtin_amdgcn_readfirstlane(ent.z);
      }
      u32x4_t wu[kU][NV], wd[kU][NV];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int64_t ro = int64_t(jj[q]) * d * E::kBytes;
        const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
        const u32x4_t* dr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + ro);
        if (q < nq) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            wu[q][v] = ur[v * kWave + lane];
            wd[q][v] = dr[v * kWave + lane];
          }
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) wu[q][v] = wd[q][v] = u32x4_t{0, 0, 0, 0};
        }
      }
      float hq[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        // x comes from LDS one 16-byte piece at a time (keeps 12 VGPRs free)
        const u32x4_t* xq = xw + kk[q] * kRowVec;
        float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const u32x4_t xv = xq[v * kWave + lane];
          lane_dot_piece<E>(wu[q][v], xv, acc4);
          __builtin_amdgcn_sched_barrier(0);
        }
        hq[q] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) hq[q] = aa[q] * wave_sum(hq[q]);
#pragma unroll
      for (int q = 0; q < kU; ++q) {
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          if (kk[q] == k) {  // wave-uniform
            const AxpyCoef<E> hc(hq[q]);
#pragma unroll
            for (int v = 0; v < NV; ++v) hc.axpy(wd[q][v], yf[k][v]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    if (act[k]) {
      u32x4_t* yr = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.y) + tk[k] * d * E::kBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(Vec<E>::pack(yf[k][v]), yr + v * kWave + lane);
    }
  }
}

// Small-batch variant (few tokens): one workgroup of kW waves per token (16;
// 8 for bf16 rows wider than 2048, whose fp32 partial row needs the 256 VGPRs
// of two waves per SIMD), the waves splitting the token's tiles into kW
// ranges, so a batch of T tokens keeps T workgroups busy instead of T/32.
// Each wave walks its range like fused_updown_kernel; the kW fp32 partial rows
// meet in LDS and are summed in ascending range order (deterministic) before
// y[t] is written once.
constexpr int kTokWaves = 16;
constexpr int kTokWavesWide = 8;  // bf16 rows wider than 2048: 256 VGPRs per wave for the fp32 partial row
constexpr int kTokList = kWave;  // list entries per wave and pass (one per slot)

template <int NV, int EB, int kW>
constexpr size_t token_lds_bytes() {
  return static_cast<size_t>(kW) * kTokList * 8 + static_cast<size_t>(kW) * NV * kWave * (16 / EB) * 4 +
         static_cast<size_t>(NV) * kWave * 16;
}

// waves per SIMD the registers must allow: 4 for the 8-wave variant of rows
// up to 4 vectors per lane (two workgroups, two tokens, share a CU), else no
// more than one workgroup needs
template <class E, int NV, int kW>
constexpr int token_waves_per_simd() { return kW < kTokWaves && NV * Vec<E>::N <= 32 ? 4 : 1; }

template <class E, int NV, int kW>
__global__ __launch_bounds__(kW * kWave, (token_waves_per_simd<E, NV, kW>())) void fused_updown_token_kernel(FusedArgs p) {
  constexpr int kN = Vec<E>::N;
  constexpr int kU = NV <= 2 ? 4 : (NV <= 4 ? 2 : 1);
  constexpr int kRow = NV * kWave * kN;  // d_model
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int2* list = reinterpret_cast<int2*>(smem) + wave * kTokList;  // this wave's entries of a pass
  float* ypart = reinterpret_cast<float*>(smem + kW * kTokList * 8);  // [kW][d]
  u32x4_t* xl = reinterpret_cast<u32x4_t*>(ypart + kW * kRow);       // x[t], shared by the waves
  const int64_t i_row = blockIdx.x;
  const int64_t n_rows = p.n_rows_dev ? static_cast<int64_t>(*p.n_rows_dev) : p.T;
  if (i_row >= n_rows) return;  // uniform over the workgroup, before any barrier
  const int64_t t = p.rows ? static_cast<int64_t>(p.rows[i_row]) : i_row;
  const int d = p.d, C = p.C, tile_n = p.tile_n;
  const int n_t = p.F / tile_n;
  const int tg = (n_t + kW - 1) / kW;
  const int b_begin = min(n_t, wave * tg), b_end = min(n_t, b_begin + tg);

  // The wave's TwELL slots, tile-major (tile b_begin + s / C, slot s % C),
  // one per lane and pass of 64: the slot's tile count, index and value are
  // loaded together, so a pass's list takes one memory round trip, not a
  // count load followed by index loads.  A slot holds an entry iff it is
  // below min(count, C); entries keep ascending (tile, slot) order.
  const int n_slots = (b_end - b_begin) * C;
  auto slot = [&](int s, int& j, float& a) -> bool {
    if (s >= n_slots) return false;
    const int q = s / C, sl = s - q * C;
    const int64_t unit = t * n_t + b_begin + q;
    const int cnt = p.count[unit];
    const int ix = p.idx[unit * C + sl];
    a = load_elem<E>(p.val, unit * C + sl);
    j = (b_begin + q) * tile_n + (ix & (tile_n - 1));
    return sl < min(cnt, C);
  };
  int j_first = 0;
  float a_first = 0.f;
  const bool v_first = slot(lane, j_first, a_first);  // issued beside the x row
  float yf[NV][kN];
  {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.x) + t * d * E::kBytes);
    for (int v = threadIdx.x; v < NV * kWave; v += kW * kWave) xl[v] = xr[v];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < kN; ++i) yf[v][i] = 0.f;
  }
  __syncthreads();
  for (int s0 = 0; s0 < n_slots; s0 += kWave) {
    int j = j_first;
    float a = a_first;
    const bool valid = s0 == 0 ? v_first : slot(s0 + lane, j, a);
    const uint64_t m = __builtin_amdgcn_ballot_w64(valid);
    const int total = static_cast<int>(__popcll(m));  // <= kTokList
    if (valid)
      list[__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u))] =
          make_int2(j, __float_as_int(a));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int e0 = 0; e0 < total; e0 += kU) {
      int jj[kU];
      float aa[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int2 ent = list[min(e0 + q, total - 1)];
        jj[q] = __builtin_amdgcn_readfirstlane(ent.x);
        aa[q] = (e0 + q < total) ? __int_as_float(__builtin_amdgcn_readfirstlane(ent.y)) : 0.f;
      }
      const int nq = min(kU, total - e0);
      u32x4_t wu[kU][NV], wd[kU][NV];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int64_t ro = int64_t(jj[q]) * d * E::kBytes;
        const u32x4_t* ur = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_up_t) + ro);
        const u32x4_t* dr = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.w_down) + ro);
        if (q < nq) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            wu[q][v] = ur[v * kWave + lane];
            wd[q][v] = dr[v * kWave + lane];
          }
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v) wu[q][v] = wd[q][v] = u32x4_t{0, 0, 0, 0};
        }
      }
      float hq[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        u32x4_t xv[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) xv[v] = xl[v * kWave + lane];
        hq[q] = aa[q] * wave_sum(lane_dot<E, NV>(wu[q], xv));
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const AxpyCoef<E> hc(hq[q]);
#pragma unroll
        for (int v = 0; v < NV; ++v) hc.axpy(wd[q][v], yf[v]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // partial rows -> LDS, then a fixed-order sum over the 16 ranges
  float* mine = ypart + wave * kRow;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < kN; i += 4)
      *reinterpret_cast<float4*>(mine + (v * kWave + lane) * kN + i) =
          make_float4(yf[v][i], yf[v][i + 1], yf[v][i + 2], yf[v][i + 3]);
  __syncthreads();
  for (int e = threadIdx.x; e < kRow; e += kW * kWave) {
    float acc = ypart[e];
#pragma unroll
    for (int w = 1; w < kW; ++w) acc += ypart[w * kRow + e];
    store_bits<E>(p.y, t * d + e, round_store<E>(acc).bits);
  }
}

template <class E, int NV, int kW>
static hipError_t launch_token_w(const FusedArgs& a, hipStream_t s) {
  constexpr size_t lds = token_lds_bytes<NV, E::kBytes, kW>();
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fused_updown_token_kernel<E, NV, kW>), hipFuncAttributeMaxDynamicSharedMemorySize,
      static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fused_updown_token_kernel<E, NV, kW>), dim3(static_cast<unsigned>(a.T)), dim3(kW * kWave), lds, s,
                     a);
  return hipGetLastError();
}

// 16 waves per token while the batch leaves CUs idle; from kTokPairT tokens
// on 8 waves, so that two tokens' workgroups share a CU (16 waves of 128 VGPRs
// fit one workgroup per CU); bf16 rows wider than 2048 always 8 waves.
constexpr int64_t kTokPairT = 512;

template <class E, int NV>
static hipError_t launch_token_t(const FusedArgs& a, hipStream_t s) {
  if constexpr (NV * Vec<E>::N <= 32) {
    if (a.T < kTokPairT) return launch_token_w<E, NV, kTokWaves>(a, s);
  }
  return launch_token_w<E, NV, kTokWavesWide>(a, s);
}

template <int NV, int TPW, int kW>
constexpr size_t sync_lds_bytes() {
  return static_cast<size_t>(kW) * TPW * NV * kWave * 16 + kW * kSyncList * 16;
}

template <class E, int NV, int TPW, int kU, int kW>
static hipError_t launch_sync_cfg(const FusedArgs& args, hipStream_t s) {
  constexpr size_t lds = sync_lds_bytes<NV, TPW, kW>();
  static_assert(lds <= 160 * 1024, "LDS of one workgroup");
  FusedArgs a = args;
  a.resident = lockstep_resident();
  const int64_t per_block = static_cast<int64_t>(kW) * TPW;
  const int64_t blocks = (a.T + per_block - 1) / per_block;
  // one launch per generation of resident workgroups, so every generation
  // starts on a free chip, its workgroups together
  const int64_t step = a.resident > 0 ? a.resident : blocks;
  for (int64_t b0 = 0; b0 < blocks; b0 += step) {
    a.blk0 = b0;
    dim3 grid(static_cast<unsigned>(blocks - b0 < step ? blocks - b0 : step));
    if constexpr (E::kBytes == 2) {
      if (a.C == 16) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&fused_updown_sync_kernel<E, NV, TPW, kU, 16, kW>),
            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((fused_updown_sync_kernel<E, NV, TPW, kU, 16, kW>), grid, dim3(kW * kWave), lds, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        continue;
      }
    }
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fused_updown_sync_kernel<E, NV, TPW, kU, 0, kW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((fused_updown_sync_kernel<E, NV, TPW, kU, 0, kW>), grid, dim3(kW * kWave), lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Tokens per wave: as many fp32 y rows as fit beside the loads in the VGPRs
// of a wave (128 at 16 waves, 256 at 8) and their x rows in LDS, and no more
// than the per-chunk list holds when one tile of each token is
// full (TPW * C <= kSyncList, so every chunk of >= 1 tile fits), but fewer when
// that would leave CUs without a workgroup (e.g. 8192 rows at d_model = 1024:
// 4 tokens per wave give 128 workgroups for 256 CUs, 2 give 256).
template <class E, int NV>
static hipError_t launch_sync_t(const FusedArgs& a, hipStream_t s) {
  constexpr int kW = NV <= 4 ? kSyncWaves : kSyncWavesWide;
  // rows per wave: their fp32 accumulators fit beside the loads, and the x rows
  // of the workgroup fit in LDS beside the entry lists
  constexpr int kRegMax = NV * Vec<E>::N <= 16 ? 4 : 2;
  constexpr int kLdsMax = static_cast<int>((160 * 1024 - kW * kSyncList * 16) / (kW * NV * kWave * 16));
  constexpr int kMax = kRegMax < kLdsMax ? kRegMax : kLdsMax;
  static_assert(kMax >= 1, "one row per wave fits");
  const int fit = kSyncList / a.C;
  const int64_t cus = lockstep_resident();
  auto fills = [&](int tpw) {
    const int64_t per = static_cast<int64_t>(kW) * tpw;
    return cus <= 0 || (a.T + per - 1) / per >= cus;
  };
  if constexpr (kMax >= 4) {
    if (fit >= 4 && fills(4)) return launch_sync_cfg<E, NV, 4, 1, kW>(a, s);
  }
  if constexpr (kMax >= 2) {
    if (fit >= 2 && fills(2)) return launch_sync_cfg<E, NV, 2, 1, kW>(a, s);
  }
  return launch_sync_cfg<E, NV, 1, 1, kW>(a, s);
}

template <class E, int NV>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.T + kWavesPerBlock - 1) / kWavesPerBlock));
  hipLaunchKernelGGL((fused_updown_kernel<E, NV, false>), grid, dim3(kWavesPerBlock * kWave), 0, s, a);
  return hipGetLastError();
}

template <class E, int NV>
static hipError_t launch_split_t(const FusedArgs& a, hipStream_t s) {
  const int64_t units = a.part_rows * a.groups;
  dim3 grid(static_cast<unsigned>((units + kWavesPerBlock - 1) / kWavesPerBlock));
  hipLaunchKernelGGL((fused_updown_kernel<E, NV, true>), grid, dim3(kWavesPerBlock * kWave), 0, s, a);
  return hipGetLastError();
}

template <class E>
static hipError_t launch_split_e(const FusedArgs& a, hipStream_t s) {
  if (a.part_rows <= 0 || a.groups <= 0) return hipSuccess;
  switch (a.d / (kWave * Vec<E>::N)) {
    case 1: return launch_split_t<E, 1>(a, s);
    case 2: return launch_split_t<E, 2>(a, s);
    case 3: return launch_split_t<E, 3>(a, s);
    case 4: return launch_split_t<E, 4>(a, s);
    case 5: return launch_split_t<E, 5>(a, s);
    case 6: return launch_split_t<E, 6>(a, s);
    case 7: return launch_split_t<E, 7>(a, s);
    case 8: return launch_split_t<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused_split(const FusedArgs& a, int dtype, hipStream_t s) {
  hipError_t e = dtype == 1 ? launch_split_e<EBf16>(a, s) : launch_split_e<EF32>(a, s);
  if (e != hipSuccess || a.part_rows <= 0 || a.groups <= 0) return e;
  return launch_splitk_reduce(a.part, a.groups, a.part_rows, a.n_rows_dev, a.rows, a.y, a.d, dtype, s);
}

// Batches below this many tokens use the one-workgroup-per-token kernel (the
// lockstep kernel would keep fewer than T/32 workgroups busy).
constexpr int64_t kSmallBatch = 2048;

// Rows wider than 4 16-byte vectors per lane: bf16 batches of kWideSyncBatch
// rows and more take the 8-wave lockstep kernel (from there two rows per wave
// fill a generation of workgroups; at 2100 rows a nearly empty second
// generation made it a third slower than a wave per token); smaller batches
// and fp32 take a wave per token.
constexpr int64_t kWideSyncBatch = 4096;

template <class E, int NV>
static hipError_t launch_wide_t(const FusedArgs& a, hipStream_t s) {
  if constexpr (E::kBytes == 2) {
    if (a.T >= kWideSyncBatch) return launch_sync_t<E, NV>(a, s);
  }
  return launch_fused_t<E, NV>(a, s);
}

template <class E>
static hipError_t launch_fused_e(const FusedArgs& a, hipStream_t s) {
  const int nv = a.d / (kWave * Vec<E>::N);
  if (a.T < kSmallBatch) {
    switch (nv) {  // NV <= 8: d_model <= 4096 in bf16 (8 waves above 2048), <= 2048 in fp32
      case 1: return launch_token_t<E, 1>(a, s);
      case 2: return launch_token_t<E, 2>(a, s);
      case 3: return launch_token_t<E, 3>(a, s);
      case 4: return launch_token_t<E, 4>(a, s);
      case 5: return launch_token_t<E, 5>(a, s);
      case 6: return launch_token_t<E, 6>(a, s);
      case 7: return launch_token_t<E, 7>(a, s);
      case 8: return launch_token_t<E, 8>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nv) {
    case 1: return launch_sync_t<E, 1>(a, s);
    case 2: return launch_sync_t<E, 2>(a, s);
    case 3: return launch_sync_t<E, 3>(a, s);
    case 4: return launch_sync_t<E, 4>(a, s);
    case 5: return launch_wide_t<E, 5>(a, s);
    case 6: return launch_wide_t<E, 6>(a, s);
    case 7: return launch_wide_t<E, 7>(a, s);
    case 8: return launch_wide_t<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused_updown(const FusedArgs& a, int dtype, hipStream_t s) {
  return dtype == 1 ? launch_fused_e<EBf16>(a, s) : launch_fused_e<EF32>(a, s);
}

}  // namespace twell
