// C ABI of libtwell: host-side validation and kernel dispatch.  Every check
// happens before any HIP call, so a bad descriptor or pointer costs nothing on
// the device and can be tested without a GPU.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>

#include "../../include/twell.h"
#include "api_internal.hpp"
#include "internal.hpp"

namespace {

constexpr int64_t kIndexLimit = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int elem_bytes(const twell_desc* d) { return d->dtype == TWELL_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.
twell_status check_desc(const twell_desc* d) {
  if (!d) return TWELL_EINVAL;
  if (d->T < 0 || d->d_model <= 0 || d->d_ff <= 0 || d->tile_n <= 0 || d->slots <= 0) return TWELL_EINVAL;
  if (d->dtype != TWELL_FP32 && d->dtype != TWELL_BF16) return TWELL_EINVAL;
  if (d->d_ff % d->tile_n != 0) return TWELL_EINVAL;
  if (d->slots > d->tile_n) return TWELL_EINVAL;
  if (d->tile_n != 64 && d->tile_n != 128) return TWELL_EUNSUPPORTED;
  if (d->dtype == TWELL_BF16) {
    if (d->d_model % 512 != 0 || d->d_model > 4096) return TWELL_EUNSUPPORTED;
  } else {
    if (d->d_model % 256 != 0 || d->d_model > 2048) return TWELL_EUNSUPPORTED;
  }
  const int64_t widest = d->d_ff > d->d_model ? d->d_ff : d->d_model;
  if (d->T > 0 && d->T > (kIndexLimit - 1) / widest) return TWELL_EUNSUPPORTED;
  return TWELL_OK;
}

twell_status check_act(const twell_act& a) {
  if (!a.count || !a.idx || !a.val) return TWELL_EINVAL;
  if (!aligned16(a.count) || !aligned16(a.idx) || !aligned16(a.val)) return TWELL_EINVAL;
  return TWELL_OK;
}

twell_status check_dense_ptr(const void* p) {
  if (!p || !aligned16(p)) return TWELL_EINVAL;
  return TWELL_OK;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace layout of the hybrid forward: router block counts, then the dense
// rows' hidden activations h [max_dense_rows x d_ff].
// Split-K factor of the dense rows' GEMMs that reduce over d_ff.
int dense_splits(const twell_desc* d) { return twell::split_k_for(d->d_ff, 128 / elem_bytes(d)); }

// Heavy ELL rows of the hybrid forward (row total > max(2 C, 2 x mean)): at
// most kHeavyCap of them are cut into heavy_groups() tile ranges each.
constexpr int64_t kHeavyCap = 1024;
int64_t heavy_cap(const twell_desc* d) { return d->T < kHeavyCap ? d->T : kHeavyCap; }
int heavy_groups(const twell_desc* d) {
  const int n_t = d->d_ff / d->tile_n;
  return n_t < 8 ? n_t : 8;
}

// Workspace layout of the hybrid forward: router block counts, the dense rows'
// hidden activations h [max_dense_rows x d_ff], the split-K partials of their
// down GEMM [splits x max_dense_rows x d_model] fp32 (splits > 1 only), then
// the light / heavy split of the ELL rows (row totals, block totals, the two
// lists, their counters) and the heavy rows' partial outputs
// [groups x heavy_cap x d_model] fp32.
struct HybridWs {
  size_t block_dense, h, part, row_total, block_total, block_heavy, light, heavy, split_n, heavy_part, total;
};
HybridWs hybrid_ws(const twell_desc* d, int64_t max_dense_rows) {
  HybridWs w{};
  const size_t T = static_cast<size_t>(d->T);
  const size_t nblk = (T + 255) / 256;
  const size_t cap = static_cast<size_t>(max_dense_rows);
  const int sp = dense_splits(d);
  w.block_dense = 0;
  w.h = align256(nblk * 4);
  w.part = w.h + align256(cap * d->d_ff * elem_bytes(d));
  size_t o = w.part + (sp > 1 ? align256(static_cast<size_t>(sp) * cap * d->d_model * 4) : 0);
  w.row_total = o;   o += align256(T * 4);
  w.block_total = o; o += align256(nblk * 4);
  w.block_heavy = o; o += align256(nblk * 4);
  w.light = o;       o += align256(T * 4);
  w.heavy = o;       o += align256(static_cast<size_t>(heavy_cap(d)) * 4);
  w.split_n = o;     o += 256;
  w.heavy_part = o;  o += align256(static_cast<size_t>(heavy_groups(d)) * heavy_cap(d) * d->d_model * 4);
  w.total = o;
  return w;
}

// Workspace layout of the backward.
struct BwdWs {
  size_t blk_hist, blk_mask, neuron_off, pairs, coef, g_d, u_d, e_d, dg_d, du_d, h_d, dx_part, row_total, block_total, block_heavy,
      light, heavy, split_n, dx_hpart, total;
};
BwdWs bwd_ws(const twell_desc* d, int64_t max_dense_rows) {
  BwdWs w{};
  const size_t T = static_cast<size_t>(d->T), F = static_cast<size_t>(d->d_ff);
  const size_t slots = T * static_cast<size_t>(d->d_ff / d->tile_n) * static_cast<size_t>(d->slots);
  const size_t cap = static_cast<size_t>(max_dense_rows), eb = static_cast<size_t>(elem_bytes(d));
  size_t o = 0;
  w.blk_hist = o;   o += align256(((T + 63) / 64) * F * 4);
  w.blk_mask = o;   o += align256(((T + 63) / 64) * F * 8);
  w.neuron_off = o; o += align256((F + 1) * 4);
  w.pairs = o;      o += align256(slots * 8);
  w.coef = o;       o += align256(slots * 8);
  w.g_d = o;        o += align256(cap * F * 4);
  w.u_d = o;        o += align256(cap * F * 4);
  w.e_d = o;        o += align256(cap * F * 4);
  w.dg_d = o;       o += align256(cap * F * eb);
  w.du_d = o;       o += align256(cap * F * eb);
  w.h_d = o;        o += align256(cap * F * eb);
  const int sp = dense_splits(d);
  w.dx_part = o;    o += sp > 1 ? align256(static_cast<size_t>(sp) * cap * static_cast<size_t>(d->d_model) * 4) : 0;
  w.row_total = o;  o += align256(T * 4);
  w.block_total = o; o += align256(((T + 255) / 256) * 4);
  w.block_heavy = o; o += align256(((T + 255) / 256) * 4);
  w.light = o;      o += align256(T * 4);
  w.heavy = o;      o += align256(static_cast<size_t>(heavy_cap(d)) * 4);
  w.split_n = o;    o += 256;
  w.dx_hpart = o;   o += align256(static_cast<size_t>(heavy_groups(d)) * heavy_cap(d) * d->d_model * 4);
  w.total = o;
  return w;
}

#define TWELL_TRY(expr)                      \
  do {                                       \
    twell_status st_ = (expr);               \
    if (st_ != TWELL_OK) return st_;         \
  } while (0)

twell_status from_hip(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_EHIP; }

}  // namespace

namespace twell {

// Workgroups of the lockstep kernels the device runs at once: one per CU
// (their LDS or VGPR footprint).  0 when the device cannot be queried: the
// launchers then issue the whole grid in one dispatch.
int lockstep_resident() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace twell

namespace twell {

twell_status hybrid_check(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                          const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                          size_t* ws_need) {
  TWELL_TRY(check_desc(d));
  if (!route || route->max_dense_rows < 0 || !ws_need) return TWELL_EINVAL;
  *ws_need = 0;
  if (d->T == 0) return TWELL_OK;
  TWELL_TRY(check_dense_ptr(x));
  TWELL_TRY(check_dense_ptr(w_gate_t));
  TWELL_TRY(check_act(act));
  TWELL_TRY(check_dense_ptr(w_up_t));
  TWELL_TRY(check_dense_ptr(w_down));
  TWELL_TRY(check_dense_ptr(y));
  if (!route->ell_rows || !route->n_rows || !route->row_kind) return TWELL_EINVAL;
  if (route->max_dense_rows > 0 && !route->dense_rows) return TWELL_EINVAL;
  if (!aligned4(route->ell_rows) || !aligned4(route->n_rows) ||
      (route->dense_rows && !aligned4(route->dense_rows)))
    return TWELL_EINVAL;
  *ws_need = hybrid_ws(d, route->max_dense_rows).total;
  return TWELL_OK;
}

twell_status hybrid_launch(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                           const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                           void* ws, void* stream) {
  const HybridWs hw = hybrid_ws(d, route->max_dense_rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);

  twell::RouteArgs r{};
  r.count = act.count;
  r.T = d->T;
  r.n_t = d->d_ff / d->tile_n;
  r.C = d->slots;
  r.cap = route->max_dense_rows;
  r.flags = route->row_kind;
  r.block_dense = reinterpret_cast<int32_t*>(wsb + hw.block_dense);
  r.ell_rows = route->ell_rows;
  r.dense_rows = route->dense_rows;
  r.n_rows = route->n_rows;
  r.row_total = reinterpret_cast<int32_t*>(wsb + hw.row_total);
  r.block_total = reinterpret_cast<int32_t*>(wsb + hw.block_total);
  r.light_rows = reinterpret_cast<int32_t*>(wsb + hw.light);
  r.heavy_rows = reinterpret_cast<int32_t*>(wsb + hw.heavy);
  r.split_n = reinterpret_cast<int32_t*>(wsb + hw.split_n);
  r.block_heavy = reinterpret_cast<int32_t*>(wsb + hw.block_heavy);
  r.heavy_cap = heavy_cap(d);
  TWELL_TRY(from_hip(twell::launch_route(r, s)));
  TWELL_TRY(from_hip(twell::launch_route_split(r, s)));

  twell::FusedArgs f{};
  f.x = x;
  f.count = act.count;
  f.idx = act.idx;
  f.val = act.val;
  f.w_up_t = w_up_t;
  f.w_down = w_down;
  f.y = y;
  f.rows = r.light_rows;
  f.n_rows_dev = r.split_n + 0;
  f.row_total = r.row_total;  // written by the route pass above
  f.T = d->T;
  f.d = d->d_model;
  f.F = d->d_ff;
  f.tile_n = d->tile_n;
  f.C = d->slots;
  TWELL_TRY(from_hip(twell::launch_fused_updown(f, d->dtype, s)));
  twell::FusedArgs fh = f;  // heavy ELL rows, cut into tile ranges
  fh.rows = r.heavy_rows;
  fh.n_rows_dev = r.split_n + 1;
  fh.groups = heavy_groups(d);
  fh.part = reinterpret_cast<float*>(wsb + hw.heavy_part);
  fh.part_rows = r.heavy_cap;
  TWELL_TRY(from_hip(twell::launch_fused_split(fh, d->dtype, s)));

  if (route->max_dense_rows == 0) return TWELL_OK;
  twell::GateUpArgs g{};
  g.x = x;
  g.w_gate_t = w_gate_t;
  g.w_up_t = w_up_t;
  g.h = wsb + hw.h;
  g.rows = route->dense_rows;
  g.n_rows_dev = route->n_rows + 1;
  g.M = route->max_dense_rows;
  g.d = d->d_model;
  g.F = d->d_ff;
  TWELL_TRY(from_hip(twell::launch_gateup(g, d->dtype, s)));
  twell::DownArgs dn{};
  dn.h = wsb + hw.h;
  dn.w_down = w_down;
  dn.y = y;
  dn.rows = route->dense_rows;
  dn.n_rows_dev = route->n_rows + 1;
  dn.M = route->max_dense_rows;
  dn.d = d->d_model;
  dn.F = d->d_ff;
  dn.splits = dense_splits(d);
  dn.part = reinterpret_cast<float*>(wsb + hw.part);
  return from_hip(twell::launch_down(dn, d->dtype, s));
}


}  // namespace twell

extern "C" {

twell_status twell_sizes(const twell_desc* d, int64_t max_dense_rows, twell_sizes_t* out) {
  TWELL_TRY(check_desc(d));
  if (!out || max_dense_rows < 0) return TWELL_EINVAL;
  const size_t T = static_cast<size_t>(d->T);
  const size_t n_t = static_cast<size_t>(d->d_ff / d->tile_n);
  const size_t C = static_cast<size_t>(d->slots);
  const size_t eb = static_cast<size_t>(elem_bytes(d));
  out->count = T * n_t * 4;
  out->idx = T * n_t * C;
  out->val = T * n_t * C * eb;
  out->ws_dense_fwd = align256(T * static_cast<size_t>(d->d_ff) * eb) +
                      static_cast<size_t>(d->d_model) * static_cast<size_t>(d->d_ff) * eb;
  const HybridWs hw = hybrid_ws(d, max_dense_rows);
  out->ws_hybrid = hw.total;
  out->ws_bwd = bwd_ws(d, max_dense_rows).total;
  out->ws_pack_classic = T * static_cast<size_t>(d->d_ff) * eb;
  return TWELL_OK;
}

twell_status twell_pack(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                        int64_t* stats, void* gate_dbg, void* stream) {
  TWELL_TRY(check_desc(d));
  if (d->T == 0) return TWELL_OK;
  TWELL_TRY(check_dense_ptr(x));
  TWELL_TRY(check_dense_ptr(w_gate_t));
  TWELL_TRY(check_act(act));
  if (stats && (reinterpret_cast<uintptr_t>(stats) & 7u)) return TWELL_EINVAL;
  if (gate_dbg && !aligned4(gate_dbg)) return TWELL_EINVAL;
  twell::PackArgs a{};
  a.x = x;
  a.w_gate_t = w_gate_t;
  a.T = d->T;
  a.d = d->d_model;
  a.F = d->d_ff;
  a.tile_n = d->tile_n;
  a.C = d->slots;
  a.count = act.count;
  a.idx = act.idx;
  a.val = act.val;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  a.gate_dbg = gate_dbg;
  return from_hip(twell::launch_gate_pack(a, d->dtype, static_cast<hipStream_t>(stream)));
}

twell_status twell_ffn_fwd(const twell_desc* d, const void* x, twell_act act, const void* w_up_t,
                           const void* w_down, void* y, void* stream) {
  TWELL_TRY(check_desc(d));
  if (d->T == 0) return TWELL_OK;
  TWELL_TRY(check_dense_ptr(x));
  TWELL_TRY(check_act(act));
  TWELL_TRY(check_dense_ptr(w_up_t));
  TWELL_TRY(check_dense_ptr(w_down));
  TWELL_TRY(check_dense_ptr(y));
  twell::FusedArgs a{};
  a.rows = nullptr;
  a.n_rows_dev = nullptr;
  a.x = x;
  a.count = act.count;
  a.idx = act.idx;
  a.val = act.val;
  a.w_up_t = w_up_t;
  a.w_down = w_down;
  a.y = y;
  a.T = d->T;
  a.d = d->d_model;
  a.F = d->d_ff;
  a.tile_n = d->tile_n;
  a.C = d->slots;
  return from_hip(twell::launch_fused_updown(a, d->dtype, static_cast<hipStream_t>(stream)));
}

twell_status twell_ffn_fwd_hybrid(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                                  const void* w_up_t, const void* w_down, void* y, const twell_route* route,
                                  void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  TWELL_TRY(twell::hybrid_check(d, x, w_gate_t, act, w_up_t, w_down, y, route, &need));
  if (d->T == 0) return TWELL_OK;
  if (!ws || !aligned16(ws) || ws_bytes < need) return TWELL_EINVAL;
  return twell::hybrid_launch(d, x, w_gate_t, act, w_up_t, w_down, y, route, ws, stream);
}

twell_status twell_ffn_bwd(const twell_desc* d, const void* x, twell_act act, const twell_route* route,
                           const void* w_gate_t, const void* w_up_t, const void* w_down, const void* dy,
                           float l1_coef, void* dx, float* dw_gate_t, float* dw_up_t, float* dw_down,
                           void* ws, size_t ws_bytes, void* stream) {
  TWELL_TRY(check_desc(d));
  if (!route || route->max_dense_rows < 0) return TWELL_EINVAL;
  TWELL_TRY(check_dense_ptr(w_gate_t));
  TWELL_TRY(check_dense_ptr(w_up_t));
  TWELL_TRY(check_dense_ptr(w_down));
  TWELL_TRY(check_dense_ptr(dw_gate_t));
  TWELL_TRY(check_dense_ptr(dw_up_t));
  TWELL_TRY(check_dense_ptr(dw_down));
  const BwdWs bw = bwd_ws(d, route->max_dense_rows);
  if (!ws || !aligned16(ws) || ws_bytes < bw.total) return TWELL_EINVAL;
  if (d->T > 0) {
    TWELL_TRY(check_dense_ptr(x));
    TWELL_TRY(check_dense_ptr(dy));
    TWELL_TRY(check_dense_ptr(dx));
    TWELL_TRY(check_act(act));
    if (!route->ell_rows || !route->n_rows) return TWELL_EINVAL;
    if (route->max_dense_rows > 0 && !route->dense_rows) return TWELL_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  twell::BwdArgs a{};
  a.x = x;
  a.dy = dy;
  a.count = act.count;
  a.idx = act.idx;
  a.val = act.val;
  a.w_gate_t = w_gate_t;
  a.w_up_t = w_up_t;
  a.w_down = w_down;
  a.ell_rows = route->ell_rows;
  a.dense_rows = route->dense_rows;
  a.n_rows = route->n_rows;
  a.T = d->T;
  a.cap = d->T > 0 ? route->max_dense_rows : 0;
  a.d = d->d_model;
  a.F = d->d_ff;
  a.tile_n = d->tile_n;
  a.C = d->slots;
  a.l1 = l1_coef;
  a.dx = dx;
  a.dw_gate_t = dw_gate_t;
  a.dw_up_t = dw_up_t;
  a.dw_down = dw_down;
  a.blk_hist = reinterpret_cast<int32_t*>(wsb + bw.blk_hist);
  a.blk_mask = reinterpret_cast<unsigned long long*>(wsb + bw.blk_mask);
  a.neuron_off = reinterpret_cast<int32_t*>(wsb + bw.neuron_off);
  a.pairs = reinterpret_cast<int2*>(wsb + bw.pairs);
  a.coef = reinterpret_cast<float2*>(wsb + bw.coef);
  a.g_d = reinterpret_cast<float*>(wsb + bw.g_d);
  a.u_d = reinterpret_cast<float*>(wsb + bw.u_d);
  a.e_d = reinterpret_cast<float*>(wsb + bw.e_d);
  a.dg_d = wsb + bw.dg_d;
  a.du_d = wsb + bw.du_d;
  a.h_d = wsb + bw.h_d;
  a.dx_splits = dense_splits(d);
  a.dx_part = reinterpret_cast<float*>(wsb + bw.dx_part);
  a.row_total = reinterpret_cast<int32_t*>(wsb + bw.row_total);
  a.block_total = reinterpret_cast<int32_t*>(wsb + bw.block_total);
  a.light_rows = reinterpret_cast<int32_t*>(wsb + bw.light);
  a.heavy_rows = reinterpret_cast<int32_t*>(wsb + bw.heavy);
  a.split_n = reinterpret_cast<int32_t*>(wsb + bw.split_n);
  a.block_heavy = reinterpret_cast<int32_t*>(wsb + bw.block_heavy);
  a.heavy_cap = heavy_cap(d);
  a.groups = heavy_groups(d);
  a.dx_hpart = reinterpret_cast<float*>(wsb + bw.dx_hpart);
  // dense rows first: their weight-gradient GEMM stores its part of dW, which
  // the ELL rows' per-neuron pass reads and adds to its own sums before its one
  // write of each row (instead of a separate read-modify-write pass over dW)
  TWELL_TRY(from_hip(twell::launch_bwd_dense(a, d->dtype, s)));
  return from_hip(twell::launch_bwd_sparse(a, d->dtype, s));
}

twell_status twell_pack_classic(const twell_desc* d, const void* x, const void* w_gate_t, twell_act act,
                                void* ws, size_t ws_bytes, void* stream) {
  TWELL_TRY(check_desc(d));
  if (d->T == 0) return TWELL_OK;
  TWELL_TRY(check_dense_ptr(x));
  TWELL_TRY(check_dense_ptr(w_gate_t));
  TWELL_TRY(check_act(act));
  TWELL_TRY(check_dense_ptr(ws));
  twell_sizes_t sz;
  TWELL_TRY(twell_sizes(d, 0, &sz));
  if (ws_bytes < sz.ws_pack_classic) return TWELL_EINVAL;
  twell::ClassicArgs a{};
  a.x = x;
  a.w_gate_t = w_gate_t;
  a.dense = ws;
  a.T = d->T;
  a.d = d->d_model;
  a.F = d->d_ff;
  a.tile_n = d->tile_n;
  a.C = d->slots;
  a.count = act.count;
  a.idx = act.idx;
  a.val = act.val;
  return from_hip(twell::launch_classic_pack(a, d->dtype, static_cast<hipStream_t>(stream)));
}

twell_status twell_dense_ffn_fwd(const twell_desc* d, const void* x, const void* w_gate_t,
                                 const void* w_up_t, const void* w_down, void* y, void* ws,
                                 size_t ws_bytes, void* stream) {
  TWELL_TRY(check_desc(d));
  if (d->T == 0) return TWELL_OK;
  TWELL_TRY(check_dense_ptr(x));
  TWELL_TRY(check_dense_ptr(w_gate_t));
  TWELL_TRY(check_dense_ptr(w_up_t));
  TWELL_TRY(check_dense_ptr(w_down));
  TWELL_TRY(check_dense_ptr(y));
  TWELL_TRY(check_dense_ptr(ws));
  twell_sizes_t sz;
  TWELL_TRY(twell_sizes(d, 0, &sz));
  if (ws_bytes < sz.ws_dense_fwd) return TWELL_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  twell::GateUpArgs g{};
  g.x = x;
  g.w_gate_t = w_gate_t;
  g.w_up_t = w_up_t;
  g.h = ws;
  g.rows = nullptr;
  g.n_rows_dev = nullptr;
  g.M = d->T;
  g.d = d->d_model;
  g.F = d->d_ff;
  twell::DownArgs dn{};
  dn.h = ws;
  dn.w_down = w_down;
  dn.w_down_t = static_cast<char*>(ws) + align256(static_cast<size_t>(d->T) * d->d_ff * elem_bytes(d));
  dn.y = y;
  dn.rows = nullptr;
  dn.n_rows_dev = nullptr;
  dn.M = d->T;
  dn.d = d->d_model;
  dn.F = d->d_ff;
  return from_hip(twell::launch_dense256(g, dn, d->dtype, s));
}

const char* twell_status_str(twell_status s) {
  switch (s) {
    case TWELL_OK: return "ok";
    case TWELL_EINVAL: return "invalid argument (descriptor, pointer, alignment or workspace size)";
    case TWELL_EUNSUPPORTED: return "shape or dtype not supported by the library";
    case TWELL_EHIP: return "HIP launch error";
    case TWELL_ESCRATCH: return "the problem needs more scratch than the allocation-free entry point holds";
  }
  return "unknown status";
}

}  // extern "C"
