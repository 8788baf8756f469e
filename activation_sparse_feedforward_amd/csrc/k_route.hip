// Hybrid row router.
//
// The TwELL page ("Sakana AI and NVIDIA introduce TwELL with CUDA kernels...",
// section "¿Qué hace distinto a TwELL frente a ELL clásico?") routes each row
// at run time either to a compact ELL store or, when the row has too many
// non-zeros, to a dense fallback.  Reading used here: a row is dense iff one
// of its tiles holds more non-zeros than the C slots (count > C), i.e. iff the
// ELL store would drop entries of that row.
//
// Two small kernels, no host synchronisation, deterministic output:
//   route_flags:   one thread per row -> flag[t] (1 = dense) and the number
//                  of dense rows of each 256-row block;
//   route_scatter: one thread per row -> the row's rank among dense rows
//                  (sum of earlier blocks + in-block scan), then ascending
//                  ell_rows / dense_rows lists and the counters.
// At most `cap` dense rows are kept (the fallback's workspace bound); dense
// rows past the cap go to the ELL list (lossy there) and are counted in
// n_rows[2] so the caller can see it.
#include "common.hpp"
#include "internal.hpp"

namespace twell {

constexpr int kRouteBlock = 256;

__global__ __launch_bounds__(kRouteBlock) void route_flags_kernel(RouteArgs p) {
  __shared__ int wsum[kRouteBlock / kWave];
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteBlock + threadIdx.x;
  __shared__ int wtot[kRouteBlock / kWave];
  int dense = 0, total = 0;
  if (t < p.T) {
    const int32_t* c = p.count + t * p.n_t;
    int mx = 0;
    for (int b = 0; b < p.n_t; ++b) {
      const int v = c[b];
      mx = max(mx, v);
      total += max(v, 0);
    }
    dense = mx > p.C ? 1 : 0;
    p.flags[t] = static_cast<uint8_t>(dense);
    if (p.row_total) p.row_total[t] = total;
  }
  int s = dense, st = total;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    s += __shfl_xor(s, o);
    st += __shfl_xor(st, o);
  }
  if ((threadIdx.x & 63) == 0) {
    wsum[threadIdx.x >> 6] = s;
    wtot[threadIdx.x >> 6] = st;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0, tt = 0;
    for (int w = 0; w < kRouteBlock / kWave; ++w) {
      tot += wsum[w];
      tt += wtot[w];
    }
    p.block_dense[blockIdx.x] = tot;
    if (p.block_total) p.block_total[blockIdx.x] = tt;
  }
}

__global__ __launch_bounds__(kRouteBlock) void route_scatter_kernel(RouteArgs p) {
  __shared__ int red[kRouteBlock / kWave];
  __shared__ int wpre[kRouteBlock / kWave];
  const int nblk = static_cast<int>((p.T + kRouteBlock - 1) / kRouteBlock);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // dense rows in earlier blocks (block 0 also totals every block)
  const int upto = blockIdx.x == 0 ? nblk : static_cast<int>(blockIdx.x);
  int part = 0;
  for (int i = threadIdx.x; i < upto; i += kRouteBlock) part += p.block_dense[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  int sum_upto = 0;
  for (int w = 0; w < kRouteBlock / kWave; ++w) sum_upto += red[w];
  const int before_block = blockIdx.x == 0 ? 0 : sum_upto;

  // in-block exclusive scan of the flags (ascending t)
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteBlock + threadIdx.x;
  const int f = t < p.T ? static_cast<int>(p.flags[t]) : 0;
  int incl = f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wpre[wave] = incl;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += wpre[w];
  const int64_t dense_before = before_block + wave_off + incl - f;
  if (t < p.T) {
    const int64_t kept_before = dense_before < p.cap ? dense_before : p.cap;
    if (f && dense_before < p.cap) {
      p.dense_rows[dense_before] = static_cast<int32_t>(t);
      p.flags[t] = 1;
    } else {
      p.ell_rows[t - kept_before] = static_cast<int32_t>(t);
      p.flags[t] = 0;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int64_t total = sum_upto;
    const int64_t kept = total < p.cap ? total : p.cap;
    p.n_rows[0] = static_cast<int32_t>(p.T - kept);
    p.n_rows[1] = static_cast<int32_t>(kept);
    p.n_rows[2] = static_cast<int32_t>(total - kept);
  }
}

// Split of the ELL list into light rows and at most heavy_cap heavy rows (row
// total > max(2 C, 2 x the batch's mean row total)).  Heavy rows would hold a
// lockstep workgroup of the fused kernel back at every chunk barrier; they are
// cut into tile ranges by launch_fused_split.  Both lists keep the ascending
// order of ell_rows (so everything downstream is deterministic): per block of
// 256 list positions, split_count counts the heavy rows and split_scatter
// places every row from the count of heavy rows before it (earlier blocks +
// in-block scan); heavy rows past the cap stay light.
__device__ __forceinline__ bool is_heavy_row(const RouteArgs& p, int64_t i, float mean) {
  const float thr = fmaxf(2.f * p.C, 2.f * mean);
  return static_cast<float>(p.row_total[p.ell_rows[i]]) > thr;
}

__device__ __forceinline__ float batch_mean_total(const RouteArgs& p) {
  __shared__ float s_mean;
  const int nblk = static_cast<int>((p.T + kRouteBlock - 1) / kRouteBlock);
  if (threadIdx.x == 0) {
    long long tot = 0;
    for (int b = 0; b < nblk; ++b) tot += p.block_total[b];
    s_mean = p.T > 0 ? static_cast<float>(static_cast<double>(tot) / static_cast<double>(p.T)) : 0.f;
  }
  __syncthreads();
  return s_mean;
}

__global__ __launch_bounds__(kRouteBlock) void route_split_count_kernel(RouteArgs p) {
  __shared__ int wsum[kRouteBlock / kWave];
  const float mean = batch_mean_total(p);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kRouteBlock + threadIdx.x;
  const int h = (i < p.n_rows[0] && is_heavy_row(p, i, mean)) ? 1 : 0;
  int sum = h;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) p.block_heavy[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__global__ __launch_bounds__(kRouteBlock) void route_split_scatter_kernel(RouteArgs p) {
  __shared__ int red[kRouteBlock / kWave];
  __shared__ int wpre[kRouteBlock / kWave];
  const float mean = batch_mean_total(p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_ell = p.n_rows[0];
  const int nblk = static_cast<int>((p.T + kRouteBlock - 1) / kRouteBlock);
  // heavy rows in earlier blocks (block 0 also totals every block)
  const int upto = blockIdx.x == 0 ? nblk : static_cast<int>(blockIdx.x);
  int part = 0;
  for (int b = threadIdx.x; b < upto; b += kRouteBlock) part += p.block_heavy[b];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  const int sum_upto = red[0] + red[1] + red[2] + red[3];
  const int64_t before_block = blockIdx.x == 0 ? 0 : sum_upto;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kRouteBlock + threadIdx.x;
  const bool live = i < n_ell;
  const int h = (live && is_heavy_row(p, i, mean)) ? 1 : 0;
  int incl = h;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wpre[wave] = incl;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += wpre[w];
  const int64_t heavy_before = before_block + wave_off + incl - h;
  if (live) {
    const int32_t t = p.ell_rows[i];
    if (h && heavy_before < p.heavy_cap)
      p.heavy_rows[heavy_before] = t;
    else
      p.light_rows[i - min(heavy_before, p.heavy_cap)] = t;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int64_t kept = min(static_cast<int64_t>(sum_upto), p.heavy_cap);
    p.split_n[0] = static_cast<int32_t>(n_ell - kept);
    p.split_n[1] = static_cast<int32_t>(kept);
  }
}

hipError_t launch_route_split(const RouteArgs& a, hipStream_t s) {
  const unsigned nblk = static_cast<unsigned>((a.T + kRouteBlock - 1) / kRouteBlock);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(route_split_count_kernel, dim3(nblk), dim3(kRouteBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_split_scatter_kernel, dim3(nblk), dim3(kRouteBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const unsigned nblk = static_cast<unsigned>((a.T + kRouteBlock - 1) / kRouteBlock);
  hipLaunchKernelGGL(route_flags_kernel, dim3(nblk), dim3(kRouteBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(kRouteBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
