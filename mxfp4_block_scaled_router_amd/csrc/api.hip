// C ABI of the MXFP4 routed-expert MoE layer: host-side validation (checked
// arithmetic, named refusals, all before any GPU work), workspace layout, the
// choice of kernel variant, and the launch sequence.
//
// Refusing an empty or overflowing shape by name before any size is used
// follows the loader rule of TensorFold PR #1050 (review and commit notes:
// EmptyShape / ShapeOverflow via checked arithmetic).
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/mxfp4_moe.h"
#include "common.h"
#include "launch.h"

using namespace mxmoe;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MXFP4_MOE_ERR_HIP;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// ---------------------------------------------------------------- shapes
// With the shared expert (MXFP4_MOE_SHARED_EXPERT) every token has one more
// slot, after its kp routed picks, on one more expert, after the Er routed
// local ones: El and k count the tables' experts and slots, shared one
// included, so everything after the top-k selection runs unchanged.
struct Shape {
  int64_t T, H, I, Eg, El, f, k;
  int64_t S;       // T * k: slots
  int64_t Er, kp;  // routed local experts, routed picks per token
  int64_t sh;      // 1 with the shared expert
  bool a4, a8, ordered;
  bool route_launch;  // route in its own launch even where gate_up could route
  // activation format of the GEMMs: 0 bf16, 1 MXFP4 (A4), 2 MXFP8 (A8)
  int af() const { return a4 ? 1 : a8 ? 2 : 0; }
  bool mx() const { return a4 || a8; }
  int64_t qdiv() const { return a8 ? 1 : 2; }  // elements per code byte
};

GemmPlan choose_plan(const Shape& s);

int check_dims(const mxfp4_moe_dims* d, int64_t top_k, bool need_k, Shape* s) {
  if (!d) return MXFP4_MOE_ERR_NULL_POINTER;
  if (d->reserved != 0) return MXFP4_MOE_ERR_BAD_ARGUMENT;
  if (d->flags & ~(MXFP4_MOE_A4 | MXFP4_MOE_DETERMINISTIC | MXFP4_MOE_SHARED_EXPERT | MXFP4_MOE_A8 |
                   MXFP4_MOE_ROUTE_LAUNCH))
    return MXFP4_MOE_ERR_BAD_FLAGS;
  if ((d->flags & MXFP4_MOE_A4) && (d->flags & MXFP4_MOE_A8)) return MXFP4_MOE_ERR_BAD_FLAGS;
  if (d->T < 0 || d->H < 0 || d->I < 0 || d->E_global < 0 || d->E_local < 0 || d->first_local < 0)
    return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->H == 0 || d->I == 0 || d->E_global == 0 || d->E_local == 0)
    return MXFP4_MOE_ERR_EMPTY_SHAPE;
  if (need_k) {
    if (top_k == 0) return MXFP4_MOE_ERR_EMPTY_SHAPE;
    if (top_k < 1 || top_k > d->E_global || top_k > 32) return MXFP4_MOE_ERR_BAD_TOP_K;
  }
  if (d->H % 128 || d->I % 128) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  int64_t last;
  if (!add_ok(d->first_local, d->E_local, &last)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (last > d->E_global) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->E_global > 512) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;  // router: 32 logits per lane of a 16-lane row
  s->T = d->T;
  s->H = d->H;
  s->I = d->I;
  s->Eg = d->E_global;
  s->sh = (d->flags & MXFP4_MOE_SHARED_EXPERT) ? 1 : 0;
  s->Er = d->E_local;
  s->El = d->E_local + s->sh;
  s->f = d->first_local;
  s->kp = need_k ? top_k : 1;
  s->k = s->kp + s->sh;
  s->a4 = (d->flags & MXFP4_MOE_A4) != 0;
  s->a8 = (d->flags & MXFP4_MOE_A8) != 0;
  s->ordered = (d->flags & MXFP4_MOE_DETERMINISTIC) != 0;
  s->route_launch = (d->flags & MXFP4_MOE_ROUTE_LAUNCH) != 0;
  // element counts that the kernels index with int64 and int32
  int64_t tmp;
  if (!mul_ok(s->T, s->k, &s->S)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (s->S > INT32_MAX / 2) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;  // slot ids and positions are int32
  if (!mul_ok(s->T, s->H, &tmp) || !mul_ok(tmp, 4, &tmp)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (!mul_ok(s->T, s->Eg, &tmp) || !mul_ok(tmp, 4, &tmp)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (!mul_ok(s->S, s->I, &tmp) || !mul_ok(tmp, 2, &tmp)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (!mul_ok(s->S, s->H, &tmp) || !mul_ok(tmp, 4, &tmp)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  int64_t per;
  if (!mul_ok(2 * s->I, s->H, &per) || !mul_ok(per, s->El, &tmp)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  // the large-tile GEMMs always use the slot-ordered combine: with many rows
  // per call, writing y and gathering it beats fp32 atomics into out32
  // (MXFP4_MOE_LARGE_ATOMIC=1, tuning builds only: keep the atomic combine)
  const char* la = tuning_env("MXFP4_MOE_LARGE_ATOMIC");
  if (choose_plan(*s).ms >= 8 && !(la && la[0] == '1')) s->ordered = true;
  return MXFP4_MOE_OK;
}

int check_clamp(float L) {
  if (L != L || !(L > 0.0f)) return MXFP4_MOE_ERR_BAD_CLAMP;
  return MXFP4_MOE_OK;
}

// ---------------------------------------------------------------- plans
// Token-tile height by the expected rows per expert, r = T*k / E_global
// (measured on MI355X with the decode and prefill layers' dims, T from 6 to
// 8192): 16-row tiles, which stream an expert's weights once per 16 rows, win
// up to r = 24 and lose from r = 36; 64-row tiles win at r = 36 and lose to
// the 128 x 512 tiles from r = 64.
constexpr int64_t kRowsPerExpert16 = 28;
constexpr int64_t kRowsPerExpert64 = 48;
// With MXFP4 activations and up to 256 expected rows per expert, 320-row
// tiles hold every expert of a routing whole (the rows an expert gets spread
// by about the square root of the mean; above 320 an expert takes two tiles).
constexpr int64_t kRowsPerExpert320 = 256;
// K-split plans take 32-row tiles from this many tokens on, where the
// activations of two row blocks fit the registers (measured: verify_b32 on
// the decode layer 143 -> 104 us; verify_b16 90 either way)
constexpr int64_t kKsplit32MinT = 64;

GemmPlan choose_plan(const Shape& s) {
  GemmPlan p;
  // the K-split kernels address activations through 32-bit buffer offsets and
  // use one wave per 512 elements of K (at most 16 waves)
  const bool ksplit_ok = s.T * s.H * 2 < (int64_t(1) << 30) && s.S * s.I * 2 < (int64_t(1) << 30) &&
                         s.H <= 8192 && s.I <= 8192 && (s.I / 16) % 4 == 0 && (s.H / 32) % 4 == 0;
  // MXFP4_MOE_PLAN=16|64|128|320 (tuning builds only) forces the token-tile height
  int forced = 0;
  if (const char* env = tuning_env("MXFP4_MOE_PLAN")) forced = atoi(env);
  // (the 64-row kernels have no MXFP8 activations: A8 takes the 128-row tiles)
  const bool lds64 = !s.a8 && (forced == 64 || (forced == 0 && s.S <= kRowsPerExpert64 * s.Eg));
  if (ksplit_ok && (forced == 16 || forced == 32 || (forced == 0 && s.S <= kRowsPerExpert16 * s.Eg))) {
    // K-split kernels; with many tokens an expert may fill several 16-row
    // tiles, each of which would stream the expert's weights: 32-row tiles
    // (two row blocks per weight slice) halve that
    p.ksplit = 1;
    const bool fit = ksplit_two_blocks_fit(s.H, s.af()) && ksplit_two_blocks_fit(s.I, s.af());
    p.ms = forced == 32 || (forced == 0 && s.T >= kKsplit32MinT && fit) ? 2 : 1;
    p.fg = 1; p.nw = 4;
  } else if (lds64) {
    // 64-token tiles with register-fed weights
    p.ms = 4; p.fg = 2; p.nw = 4;
  } else if (s.a4 && (forced == 0 || forced == 320) && s.S <= kRowsPerExpert320 * s.Eg &&
             tile_fits(s.af(), 320, s.H) && tile_fits(s.af(), 320, s.I)) {
    // MXFP4 activations, experts expected to hold at most 256 rows: 320-row
    // tiles, one per expert, so each expert's weights stream once.  Where
    // their LDS fits (K a multiple of 512, K/32 <= 128), the direct-weight
    // 320 x 256 tiles for both GEMMs (weights straight into registers; A4
    // prefill shape on MI355X: gate_up 455 -> 390 us, down 283 -> 246 us,
    // step 0.83 -> 0.72 ms); otherwise gate_up on 320 x 128 tiles through the
    // LDS ring and down on 128 x 512 tiles (every activation row of a 320-row
    // tile re-read by each 128-row weight block: 1.2x slower there).  MXFP8
    // activations stay on 128-row tiles (their 320-row stages leave too few
    // slots: 1.3x slower).  MXFP4_MOE_DW (tuning builds only) = 0: no
    // direct-weight tiles, 1: gate_up only, 2: both.
    p.ms = 20; p.fg = 0; p.nw = 4;
    p.ms_dn = 8;
    int dw = 2;
    if (const char* env = tuning_env("MXFP4_MOE_DW")) dw = atoi(env);
    if (dw >= 1 && tile_fits(s.af(), 320, s.H, true)) p.dw = 1;
    if (dw >= 2 && tile_fits(s.af(), 320, s.I, true)) {
      p.ms_dn = 20;
      p.dw_dn = 1;
    }
  } else {
    // 128-token x 512-weight-row tiles staged through LDS
    p.ms = 8; p.fg = 0; p.nw = 4;
  }
  return p;
}

int64_t max_tiles(const Shape& s, int mt) {
  int64_t e = s.El < s.S ? s.El : s.S;
  return e + s.S / mt;
}

// ---------------------------------------------------------------- workspace
struct Layout {
  size_t ids, w, lexp, rank, sorted, inv, chunk_cnt, counts, offsets, tile1, tile2, tiles1, tiles2;
  size_t pos_tok, pos_w, tile_tok, dn_desc;
  size_t act, out32, ybuf, xq, xs, actq, acts;
  size_t total;
};

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Down workgroups whose share descriptors the workspace holds (16-row plan
// with the routing inside gate_up; a larger down grid reads the tile table).
constexpr int kMaxDownDesc = 4096;

Layout layout_of(const Shape& s) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  const size_t S = (size_t)s.S, El = (size_t)s.El;
  L.ids = take(S * 4);
  L.w = take(S * 4);
  L.lexp = take(S * 4);
  L.rank = take(S * 4);
  L.sorted = take(S * 4);
  L.inv = take(S * 4);
  L.chunk_cnt = take(((S + 63) / 64) * El * 4);
  L.counts = take(El * 4);
  L.offsets = take((El + 1) * 4);
  L.tile1 = take((El + 1) * 4);
  L.tile2 = take((El + 1) * 4);
  {
    const GemmPlan p = choose_plan(s);
    const size_t nt = (size_t)(max_tiles(s, 16 * p.ms) > max_tiles(s, 16 * p.down_ms())
                                   ? max_tiles(s, 16 * p.ms) : max_tiles(s, 16 * p.down_ms()));
    L.tiles1 = take(nt * 16);
    L.tiles2 = take(nt * 16);
    L.tile_tok = p.ksplit ? take(nt * 16 * p.ms * 4) : 0;
    L.dn_desc = p.ksplit ? take((size_t)kMaxDownDesc * 32) : 0;
  }
  L.pos_tok = take(S * 4);
  L.pos_w = take(S * 4);
  L.act = take(S * (size_t)s.I * 2);
  L.out32 = s.ordered ? 0 : take((size_t)s.T * (size_t)s.H * 4);
  L.ybuf = s.ordered ? take(S * (size_t)s.H * 4) : 0;
  if (s.mx()) {
    L.xq = take((size_t)s.T * (size_t)s.H / (size_t)s.qdiv());
    L.xs = take((size_t)s.T * (size_t)s.H / 32);
    L.actq = take(S * (size_t)s.I / (size_t)s.qdiv());
    L.acts = take(S * (size_t)s.I / 32);
  } else {
    L.xq = L.xs = L.actq = L.acts = 0;
  }
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- device
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = (int)e;
    return MXFP4_MOE_ERR_UNSUPPORTED_DEVICE;
  }
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 1) return MXFP4_MOE_OK;
    if (g_dev_ok[dev] == -1) return MXFP4_MOE_ERR_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return MXFP4_MOE_ERR_UNSUPPORTED_DEVICE;
  }
  bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_ok[dev] = ok ? 1 : -1;
  }
  return ok ? MXFP4_MOE_OK : MXFP4_MOE_ERR_UNSUPPORTED_DEVICE;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(base) + off);
}

RouteArgs route_args(const Shape& s, const float* logits, void* ws, const Layout& L, int mt1, int mt2) {
  RouteArgs r;
  r.logits = logits;
  r.T = s.T;
  r.E_global = (int32_t)s.Eg;
  r.E_local = (int32_t)s.El;
  r.E_route = (int32_t)s.Er;
  r.picks = (int32_t)s.kp;
  r.first_local = (int32_t)s.f;
  r.top_k = (int32_t)s.k;
  r.mt1 = mt1;
  r.mt2 = mt2;
  r.ids = at<int32_t>(ws, L.ids);
  r.w = at<float>(ws, L.w);
  r.lexp = at<int32_t>(ws, L.lexp);
  r.rank = at<int32_t>(ws, L.rank);
  r.chunk_cnt = at<int32_t>(ws, L.chunk_cnt);
  r.counts = at<int32_t>(ws, L.counts);
  r.offsets = at<int32_t>(ws, L.offsets);
  r.tile_off1 = at<int32_t>(ws, L.tile1);
  r.tile_off2 = at<int32_t>(ws, L.tile2);
  r.tiles1 = at<int4>(ws, L.tiles1);
  r.tiles2 = at<int4>(ws, L.tiles2);
  r.pos_tok = at<int32_t>(ws, L.pos_tok);
  r.pos_w = at<float>(ws, L.pos_w);
  r.tile_tok = L.tile_tok ? at<int32_t>(ws, L.tile_tok) : nullptr;
  r.sorted = at<int32_t>(ws, L.sorted);
  r.inv = at<int32_t>(ws, L.inv);
  r.xmap = nullptr;
  return r;
}

int check_forward_args(const mxfp4_moe_dims* d, const void* x, const float* logits, const uint8_t* w13,
                       const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s, int32_t top_k,
                       float clamp_limit, void* out, void* ws, size_t ws_bytes, Shape* s, Layout* L) {
  int st = check_dims(d, top_k, true, s);
  if (st) return st;
  st = check_clamp(clamp_limit);
  if (st) return st;
  // x, logits and out may be NULL only when there are no tokens
  if (!w13 || !w13s || !w2 || !w2s || !ws) return MXFP4_MOE_ERR_NULL_POINTER;
  if (s->T > 0 && (!x || !logits || !out)) return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(w13s, 16) || !aligned(w2, 16) ||
      !aligned(w2s, 16) || !aligned(out, 16) || !aligned(ws, 256) || !aligned(logits, 4))
    return MXFP4_MOE_ERR_MISALIGNED;
  *L = layout_of(*s);
  if (ws_bytes < L->total) return MXFP4_MOE_ERR_WORKSPACE_TOO_SMALL;
  return MXFP4_MOE_OK;
}

// The experts kept in bf16 (n > 0), or null.
int check_bf16_experts(const Shape& s, const mxfp4_moe_bf16_experts* bx) {
  if (!bx) return MXFP4_MOE_ERR_NULL_POINTER;
  if (bx->n < 0 || bx->n > s.El) return MXFP4_MOE_ERR_BAD_ARGUMENT;
  if (bx->n == 0) return MXFP4_MOE_OK;
  if (!bx->expert_map || !bx->w13 || !bx->w2) return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(bx->expert_map, 4) || !aligned(bx->w13, 16) || !aligned(bx->w2, 16))
    return MXFP4_MOE_ERR_MISALIGNED;
  return MXFP4_MOE_OK;
}

XArgs x_args(const Shape& s, const RouteArgs& r, const mxfp4_moe_bf16_experts& bx, float clamp_limit) {
  XArgs xa{};
  xa.xmap = bx.expert_map;
  xa.E_local = (int32_t)s.El;
  xa.n = (int32_t)bx.n;
  xa.counts = r.counts;
  xa.offsets = r.offsets;
  xa.pos_tok = r.pos_tok;
  xa.pos_w = r.pos_w;
  xa.T = s.T;
  xa.rows_per_expert = s.S / s.Eg;
  xa.clamp_limit = clamp_limit;
  return xa;
}

int run_forward(const Shape& s, const Layout& L, const void* x, const float* logits, const uint8_t* w13,
                const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s, float clamp_limit, void* out,
                void* ws, hipStream_t stream, float* out32_copy = nullptr,
                hipEvent_t* events = nullptr, const mxfp4_moe_bf16_experts* bx = nullptr) {
  if (s.T == 0) return MXFP4_MOE_OK;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(events[i], stream) : hipSuccess;
  };
  if (hipError_t me = mark(0); me != hipSuccess) return hip_fail(me);
  const GemmPlan plan = choose_plan(s);
  const int mt = 16 * plan.ms, mt_dn = 16 * plan.down_ms();
  RouteArgs r = route_args(s, logits, ws, L, mt, mt_dn);
  // experts kept in bf16 get no MXFP4 tiles; their own kernels follow each GEMM
  const bool has_x = bx && bx->n > 0;
  if (has_x) r.xmap = bx->expert_map;
  // few tokens on the 16-row plan: the gate_up kernel routes them itself
  const bool fused_route = plan.ksplit && plan.ms == 1 && max_tiles(s, mt) > 0 && route_fusable(r) &&
                           !s.route_launch;
  hipError_t e = fused_route ? hipSuccess : launch_route(r, stream);
  if (e != hipSuccess) return hip_fail(e);

  if (s.mx()) {
    QuantArgs q;
    q.in = x;
    q.in_dtype = 0;
    q.rows = s.T;
    q.K = s.H;
    q.in_row_stride = s.H;
    q.codes = at<uint8_t>(ws, L.xq);
    q.scales = at<uint8_t>(ws, L.xs);
    q.fp8 = s.a8 ? 1 : 0;
    e = launch_quantize(q, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if ((e = mark(1)) != hipSuccess) return hip_fail(e);

  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.sorted = r.sorted;
  g.counts = r.counts;
  g.offsets = r.offsets;
  g.route_w = r.w;
  g.pos_tok = r.pos_tok;
  g.pos_w = r.pos_w;
  g.tile_tok = r.tile_tok;
  g.top_k = (int32_t)s.k;
  g.E_local = (int32_t)s.El;
  g.clamp_limit = clamp_limit;
  g.tile_ms = plan.ksplit ? plan.ms : 0;
  // 16-row tiles with many tokens: hot experts span several tiles, whose
  // units find the expert's weight slices in L2 when they are loaded cached
  // (measured, ep_share: gate_up 61.4 -> 52.3 us; decode, one tile per
  // expert, keeps the non-temporal loads: 58.5 vs 65.3 us cached)
  g.wcache = plan.ksplit && plan.ms == 1 && s.T >= kKsplit32MinT ? 1 : 0;
  // gate_up
  g.a_bf16 = reinterpret_cast<const uint16_t*>(x);
  g.a_rows = s.T;
  g.a_codes = s.mx() ? at<uint8_t>(ws, L.xq) : nullptr;
  g.a_scales = s.mx() ? at<uint8_t>(ws, L.xs) : nullptr;
  g.w_codes = w13;
  g.w_scales = w13s;
  g.tile_off = r.tile_off1;
  g.tiles = r.tiles1;
  g.K = s.H;
  g.N = 2 * s.I;
  g.act = at<uint16_t>(ws, L.act);
  g.zero_buf = s.ordered ? nullptr : at<float>(ws, L.out32);
  g.zero_n = s.ordered ? 0 : s.T * s.H;
  if (fused_route && r.mt1 == r.mt2) {
    // gate_up's first workgroup writes the down shares (same tile table)
    GemmArgs gd = g;
    gd.K = s.I;
    gd.N = s.H;
    int grid = 0, fb = 0, cus = 0;
    float c = 0.f;
    e = down_ksplit_shares(gd, max_tiles(s, mt), s.af(), s.ordered, &grid, &fb, &cus, &c);
    if (e != hipSuccess) return hip_fail(e);
    if (grid > 0 && grid <= kMaxDownDesc) {
      g.dn_desc = at<int4>(ws, L.dn_desc);
      g.dn_grid = grid;
      g.dn_fb = fb;
      g.dn_cus = cus;
      g.dn_c = c;
    }
  }
  e = plan.ksplit    ? launch_gate_up_ksplit(g, fused_route ? &r : nullptr, max_tiles(s, mt), s.af(), stream)
      : plan.ms >= 8 ? launch_gate_up_tile(g, max_tiles(s, mt), s.af(), mt, plan.dw, stream)
                     : launch_gate_up(g, plan, max_tiles(s, mt), s.a4, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (has_x) {
    XArgs xa = x_args(s, r, *bx, clamp_limit);
    xa.a = reinterpret_cast<const uint16_t*>(x);
    xa.w = reinterpret_cast<const uint16_t*>(bx->w13);
    xa.K = s.H;
    xa.N = 2 * s.I;
    xa.act = g.act;
    e = launch_bf16x_gate_up(xa, stream);
    if (e != hipSuccess) return hip_fail(e);
  }

  if (s.mx()) {
    QuantArgs q;
    q.in = at<uint16_t>(ws, L.act);
    q.in_dtype = 0;
    q.rows = s.S;
    q.K = s.I;
    q.in_row_stride = s.I;
    q.codes = at<uint8_t>(ws, L.actq);
    q.scales = at<uint8_t>(ws, L.acts);
    q.fp8 = s.a8 ? 1 : 0;
    e = launch_quantize(q, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if ((e = mark(2)) != hipSuccess) return hip_fail(e);

  // down + combine
  g.a_bf16 = at<uint16_t>(ws, L.act);
  g.a_rows = s.S;
  g.a_codes = s.mx() ? at<uint8_t>(ws, L.actq) : nullptr;
  g.a_scales = s.mx() ? at<uint8_t>(ws, L.acts) : nullptr;
  g.w_codes = w2;
  g.w_scales = w2s;
  g.tile_off = r.tile_off2;
  g.tiles = r.tiles2;
  g.K = s.I;
  g.N = s.H;
  g.zero_buf = nullptr;
  g.zero_n = 0;
  g.out32 = s.ordered ? nullptr : at<float>(ws, L.out32);
  g.ybuf = s.ordered ? at<float>(ws, L.ybuf) : nullptr;
  e = plan.ksplit    ? launch_down_ksplit(g, max_tiles(s, mt), s.af(), s.ordered, stream)
      : plan.ms >= 8 ? launch_down_tile(g, max_tiles(s, mt_dn), s.af(), mt_dn, plan.dw_dn, s.ordered, stream)
                     : launch_down(g, plan, max_tiles(s, mt), s.a4, s.ordered, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (has_x) {
    XArgs xa = x_args(s, r, *bx, clamp_limit);
    xa.a = at<uint16_t>(ws, L.act);
    xa.w = reinterpret_cast<const uint16_t*>(bx->w2);
    xa.K = s.I;
    xa.N = s.H;
    xa.out32 = g.out32;
    xa.ybuf = g.ybuf;
    e = launch_bf16x_down(xa, s.ordered, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if ((e = mark(3)) != hipSuccess) return hip_fail(e);

  CombineArgs c;
  c.ybuf = g.ybuf;
  c.out32 = g.out32;
  c.route_w = r.w;
  c.inv = r.inv;
  c.T = s.T;
  c.H = s.H;
  c.top_k = (int32_t)s.k;
  c.out = reinterpret_cast<uint16_t*>(out);
  c.out32_copy = s.ordered ? out32_copy : nullptr;
  e = launch_combine(c, s.ordered, stream);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = mark(4)) != hipSuccess) return hip_fail(e);
  if (out32_copy && !s.ordered) {
    e = launch_copy_rows(g.out32, out32_copy, s.T * s.H * 4, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return MXFP4_MOE_OK;
}

// Copies of the intermediates the caller asked for (NULL: skipped).
int copy_intermediates(const Shape& s, const Layout& L, void* ws, void* act, uint8_t* actq, uint8_t* acts,
                       uint8_t* xq, uint8_t* xs, hipStream_t stream) {
  if (s.T == 0) return MXFP4_MOE_OK;
  hipError_t e = hipSuccess;
  if (act) e = launch_copy_rows(at<uint8_t>(ws, L.act), act, s.S * s.I * 2, stream);
  if (e == hipSuccess && s.mx() && actq)
    e = launch_copy_rows(at<uint8_t>(ws, L.actq), actq, s.S * s.I / s.qdiv(), stream);
  if (e == hipSuccess && s.mx() && acts) e = launch_copy_rows(at<uint8_t>(ws, L.acts), acts, s.S * s.I / 32, stream);
  if (e == hipSuccess && s.mx() && xq) e = launch_copy_rows(at<uint8_t>(ws, L.xq), xq, s.T * s.H / s.qdiv(), stream);
  if (e == hipSuccess && s.mx() && xs) e = launch_copy_rows(at<uint8_t>(ws, L.xs), xs, s.T * s.H / 32, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MXFP4_MOE_OK;
}

// ---------------------------------------------------------------- scratch
// The workspace of mxfp4_moe_forward_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in for
// the device symbol): the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) uint8_t scratch[MXFP4_MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of scratch on each device (null: not looked up yet)

int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return MXFP4_MOE_ERR_UNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MXFP4_MOE_OK;
}

}  // namespace

// ==================================================================== ABI
extern "C" {

int mxfp4_moe_abi_version(void) { return MXFP4_MOE_ABI_VERSION; }

int mxfp4_moe_last_hip_error(void) { return g_last_hip_error; }

const char* mxfp4_moe_status_string(int status) {
  switch (status) {
    case MXFP4_MOE_OK: return "MXFP4_MOE_OK";
    case MXFP4_MOE_ERR_NULL_POINTER: return "MXFP4_MOE_ERR_NULL_POINTER";
    case MXFP4_MOE_ERR_EMPTY_SHAPE: return "MXFP4_MOE_ERR_EMPTY_SHAPE";
    case MXFP4_MOE_ERR_SHAPE_OVERFLOW: return "MXFP4_MOE_ERR_SHAPE_OVERFLOW";
    case MXFP4_MOE_ERR_UNSUPPORTED_SHAPE: return "MXFP4_MOE_ERR_UNSUPPORTED_SHAPE";
    case MXFP4_MOE_ERR_BAD_TOP_K: return "MXFP4_MOE_ERR_BAD_TOP_K";
    case MXFP4_MOE_ERR_BAD_CLAMP: return "MXFP4_MOE_ERR_BAD_CLAMP";
    case MXFP4_MOE_ERR_WORKSPACE_TOO_SMALL: return "MXFP4_MOE_ERR_WORKSPACE_TOO_SMALL";
    case MXFP4_MOE_ERR_MISALIGNED: return "MXFP4_MOE_ERR_MISALIGNED";
    case MXFP4_MOE_ERR_UNSUPPORTED_DEVICE: return "MXFP4_MOE_ERR_UNSUPPORTED_DEVICE";
    case MXFP4_MOE_ERR_HIP: return "MXFP4_MOE_ERR_HIP";
    case MXFP4_MOE_ERR_BAD_FLAGS: return "MXFP4_MOE_ERR_BAD_FLAGS";
    case MXFP4_MOE_ERR_BAD_ARGUMENT: return "MXFP4_MOE_ERR_BAD_ARGUMENT";
    case MXFP4_MOE_ERR_SCRATCH_LIMIT: return "MXFP4_MOE_ERR_SCRATCH_LIMIT";
    default: return "MXFP4_MOE_ERR_UNKNOWN";
  }
}

int mxfp4_moe_preshuffled_bytes(const mxfp4_moe_dims* d, size_t* w13_bytes, size_t* w13_scale_bytes,
                                size_t* w2_bytes, size_t* w2_scale_bytes) {
  Shape s;
  int st = check_dims(d, 1, false, &s);
  if (st) return st;
  if (!w13_bytes || !w13_scale_bytes || !w2_bytes || !w2_scale_bytes) return MXFP4_MOE_ERR_NULL_POINTER;
  *w13_bytes = (size_t)(s.El * codes_per_expert(2 * s.I, s.H));
  *w13_scale_bytes = (size_t)(s.El * scales_per_expert(2 * s.I, s.H));
  *w2_bytes = (size_t)(s.El * codes_per_expert(s.H, s.I));
  *w2_scale_bytes = (size_t)(s.El * scales_per_expert(s.H, s.I));
  return MXFP4_MOE_OK;
}

int mxfp4_moe_preshuffle(const mxfp4_moe_dims* d, const uint8_t* canon_w13, const uint8_t* canon_w13s,
                         const uint8_t* canon_w2, const uint8_t* canon_w2s, uint8_t* w13, uint8_t* w13s,
                         uint8_t* w2, uint8_t* w2s, hipStream_t stream) {
  Shape s;
  int st = check_dims(d, 1, false, &s);
  if (st) return st;
  if (!canon_w13 || !canon_w13s || !canon_w2 || !canon_w2s || !w13 || !w13s || !w2 || !w2s)
    return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(canon_w13, 16) || !aligned(canon_w2, 16) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(w13s, 4) || !aligned(w2s, 4))
    return MXFP4_MOE_ERR_MISALIGNED;
  st = check_device();
  if (st) return st;
  PreshuffleArgs p;
  p.canon_codes = canon_w13;
  p.canon_scales = canon_w13s;
  p.codes = w13;
  p.scales = w13s;
  p.E = s.El;
  p.N = 2 * s.I;
  p.K = s.H;
  p.interleave_gate_up = 1;
  hipError_t e = launch_preshuffle(p, stream);
  if (e != hipSuccess) return hip_fail(e);
  p.canon_codes = canon_w2;
  p.canon_scales = canon_w2s;
  p.codes = w2;
  p.scales = w2s;
  p.N = s.H;
  p.K = s.I;
  p.interleave_gate_up = 0;
  e = launch_preshuffle(p, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MXFP4_MOE_OK;
}

int mxfp4_moe_quantize_preshuffle(const mxfp4_moe_dims* d, const void* w13, const void* w2, int32_t in_dtype,
                                  uint8_t* w13_out, uint8_t* w13s_out, uint8_t* w2_out, uint8_t* w2s_out,
                                  hipStream_t stream) {
  Shape s;
  int st = check_dims(d, 1, false, &s);
  if (st) return st;
  if (in_dtype != MXFP4_MOE_DTYPE_BF16 && in_dtype != MXFP4_MOE_DTYPE_F32) return MXFP4_MOE_ERR_BAD_ARGUMENT;
  int64_t n, bytes;
  if (!mul_ok(2 * s.I, s.H, &n) || !mul_ok(n, s.El, &n) || !mul_ok(n, 4, &bytes)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (!w13 || !w2 || !w13_out || !w13s_out || !w2_out || !w2s_out) return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13_out, 16) || !aligned(w2_out, 16) ||
      !aligned(w13s_out, 4) || !aligned(w2s_out, 4))
    return MXFP4_MOE_ERR_MISALIGNED;
  st = check_device();
  if (st) return st;
  QuantPreshuffleArgs q;
  q.in = w13;
  q.in_dtype = in_dtype;
  q.codes = w13_out;
  q.scales = w13s_out;
  q.E = s.El;
  q.N = 2 * s.I;
  q.K = s.H;
  q.interleave_gate_up = 1;
  hipError_t e = launch_quantize_preshuffle(q, stream);
  if (e != hipSuccess) return hip_fail(e);
  q.in = w2;
  q.codes = w2_out;
  q.scales = w2s_out;
  q.N = s.H;
  q.K = s.I;
  q.interleave_gate_up = 0;
  e = launch_quantize_preshuffle(q, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MXFP4_MOE_OK;
}

int mxfp4_moe_workspace_bytes(const mxfp4_moe_dims* d, int32_t top_k, size_t* bytes) {
  Shape s;
  int st = check_dims(d, top_k, true, &s);
  if (st) return st;
  if (!bytes) return MXFP4_MOE_ERR_NULL_POINTER;
  *bytes = layout_of(s).total;
  return MXFP4_MOE_OK;
}

int mxfp4_moe_plan(const mxfp4_moe_dims* d, int32_t top_k, int32_t* tile_rows, int32_t* ordered_combine) {
  Shape s;
  int st = check_dims(d, top_k, true, &s);
  if (st) return st;
  if (!tile_rows || !ordered_combine) return MXFP4_MOE_ERR_NULL_POINTER;
  *tile_rows = 16 * choose_plan(s).ms;
  *ordered_combine = s.ordered ? 1 : 0;
  return MXFP4_MOE_OK;
}

int mxfp4_moe_forward(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                      const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s,
                      int32_t top_k, float clamp_limit, void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  Shape s;
  Layout L;
  int st = check_forward_args(d, x, router_logits, w13, w13s, w2, w2s, top_k, clamp_limit, out, workspace,
                              workspace_bytes, &s, &L);
  if (st) return st;
  st = check_device();
  if (st) return st;
  return run_forward(s, L, x, router_logits, w13, w13s, w2, w2s, clamp_limit, out, workspace, stream);
}

int mxfp4_moe_forward_noalloc(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                              const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s,
                              int32_t top_k, float clamp_limit, void* out, hipStream_t stream) {
  Shape s;
  int st = check_dims(d, top_k, true, &s);
  if (st) return st;
  const Layout L = layout_of(s);
  if (L.total > (size_t)MXFP4_MOE_NOALLOC_SCRATCH_BYTES) return MXFP4_MOE_ERR_SCRATCH_LIMIT;
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  Layout L2;
  st = check_forward_args(d, x, router_logits, w13, w13s, w2, w2s, top_k, clamp_limit, out, ws,
                          (size_t)MXFP4_MOE_NOALLOC_SCRATCH_BYTES, &s, &L2);
  if (st) return st;
  return run_forward(s, L2, x, router_logits, w13, w13s, w2, w2s, clamp_limit, out, ws, stream);
}

int mxfp4_moe_forward_timed(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                            const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s,
                            int32_t top_k, float clamp_limit, void* out, void* workspace,
                            size_t workspace_bytes, hipEvent_t* events, hipStream_t stream) {
  Shape s;
  Layout L;
  int st = check_forward_args(d, x, router_logits, w13, w13s, w2, w2s, top_k, clamp_limit, out, workspace,
                              workspace_bytes, &s, &L);
  if (st) return st;
  if (!events) return MXFP4_MOE_ERR_NULL_POINTER;
  for (int i = 0; i < 5; ++i)
    if (!events[i]) return MXFP4_MOE_ERR_NULL_POINTER;
  st = check_device();
  if (st) return st;
  return run_forward(s, L, x, router_logits, w13, w13s, w2, w2s, clamp_limit, out, workspace, stream, nullptr,
                     events);
}

int mxfp4_moe_forward_mixed(const mxfp4_moe_dims* d, const mxfp4_moe_bf16_experts* bx, const void* x,
                            const float* router_logits, const uint8_t* w13, const uint8_t* w13s,
                            const uint8_t* w2, const uint8_t* w2s, int32_t top_k, float clamp_limit,
                            void* out, void* workspace, size_t workspace_bytes, void* act, uint8_t* actq,
                            uint8_t* acts, uint8_t* xq, uint8_t* xs, float* out32, hipStream_t stream) {
  Shape s;
  Layout L;
  int st = check_forward_args(d, x, router_logits, w13, w13s, w2, w2s, top_k, clamp_limit, out, workspace,
                              workspace_bytes, &s, &L);
  if (st) return st;
  st = check_bf16_experts(s, bx);
  if (st) return st;
  if (!aligned(out32, 16) || !aligned(act, 16)) return MXFP4_MOE_ERR_MISALIGNED;
  st = check_device();
  if (st) return st;
  st = run_forward(s, L, x, router_logits, w13, w13s, w2, w2s, clamp_limit, out, workspace, stream, out32,
                   nullptr, bx);
  if (st) return st;
  return copy_intermediates(s, L, workspace, act, actq, acts, xq, xs, stream);
}

int mxfp4_moe_preshuffle_fused(const mxfp4_moe_dims* d, const uint8_t* excluded, const uint8_t* w13_fused,
                               const uint8_t* w13s_fused, const uint8_t* w2_fused, const uint8_t* w2s_fused,
                               uint8_t* w13, uint8_t* w13s, uint8_t* w2, uint8_t* w2s, void* w13_bf16,
                               void* w2_bf16, int32_t* expert_map, hipStream_t stream) {
  Shape s;
  int st = check_dims(d, 1, false, &s);
  if (st) return st;
  if (!excluded || !w13_fused || !w2_fused || !w13 || !w13s || !w2 || !w2s || !expert_map)
    return MXFP4_MOE_ERR_NULL_POINTER;
  if (s.El > kExpertMapMax) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  ExpertMapArgs m{};
  m.E = (int32_t)s.El;
  int64_t n = 0;
  for (int64_t e = 0; e < s.El; ++e) {
    if (excluded[e] > 1) return MXFP4_MOE_ERR_BAD_ARGUMENT;
    if (excluded[e]) {
      m.bits[e >> 5] |= 1u << (e & 31);
      ++n;
    }
  }
  if (n < s.El && (!w13s_fused || !w2s_fused)) return MXFP4_MOE_ERR_NULL_POINTER;
  if (n > 0 && (!w13_bf16 || !w2_bf16)) return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(w13_fused, 16) || !aligned(w2_fused, 16) || !aligned(w13s_fused, 16) || !aligned(w2s_fused, 16) ||
      !aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13s, 4) || !aligned(w2s, 4) || !aligned(w13_bf16, 16) ||
      !aligned(w2_bf16, 16) || !aligned(expert_map, 4))
    return MXFP4_MOE_ERR_MISALIGNED;
  st = check_device();
  if (st) return st;
  // per expert: packed codes (N K / 2 bytes) + scales (N K / 32), or bf16 (N K * 2)
  const int64_t n13 = 2 * s.I * s.H, n2 = s.H * s.I;
  int64_t o13 = 0, o2 = 0, so13 = 0, so2 = 0, j = 0;
  for (int64_t e = 0; e < s.El; ++e) {
    hipError_t err;
    if (excluded[e]) {
      err = launch_copy_rows(w13_fused + o13, static_cast<uint8_t*>(w13_bf16) + j * n13 * 2, n13 * 2, stream);
      if (err == hipSuccess)
        err = launch_copy_rows(w2_fused + o2, static_cast<uint8_t*>(w2_bf16) + j * n2 * 2, n2 * 2, stream);
      o13 += n13 * 2;
      o2 += n2 * 2;
      ++j;
    } else {
      PreshuffleArgs p;
      p.canon_codes = w13_fused + o13;
      p.canon_scales = w13s_fused + so13;
      p.codes = w13 + e * codes_per_expert(2 * s.I, s.H);
      p.scales = w13s + e * scales_per_expert(2 * s.I, s.H);
      p.E = 1;
      p.N = 2 * s.I;
      p.K = s.H;
      p.interleave_gate_up = 1;
      err = launch_preshuffle(p, stream);
      if (err == hipSuccess) {
        p.canon_codes = w2_fused + o2;
        p.canon_scales = w2s_fused + so2;
        p.codes = w2 + e * codes_per_expert(s.H, s.I);
        p.scales = w2s + e * scales_per_expert(s.H, s.I);
        p.N = s.H;
        p.K = s.I;
        p.interleave_gate_up = 0;
        err = launch_preshuffle(p, stream);
      }
      o13 += n13 / 2;
      o2 += n2 / 2;
      so13 += n13 / 32;
      so2 += n2 / 32;
    }
    if (err != hipSuccess) return hip_fail(err);
  }
  hipError_t err = launch_expert_map(m, expert_map, stream);
  if (err != hipSuccess) return hip_fail(err);
  return MXFP4_MOE_OK;
}

int mxfp4_moe_forward_debug(const mxfp4_moe_dims* d, const void* x, const float* router_logits,
                            const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2, const uint8_t* w2s,
                            int32_t top_k, float clamp_limit, void* out, void* workspace,
                            size_t workspace_bytes, void* act, uint8_t* actq, uint8_t* acts, uint8_t* xq,
                            uint8_t* xs, float* out32, hipStream_t stream) {
  Shape s;
  Layout L;
  int st = check_forward_args(d, x, router_logits, w13, w13s, w2, w2s, top_k, clamp_limit, out, workspace,
                              workspace_bytes, &s, &L);
  if (st) return st;
  if (!act) return MXFP4_MOE_ERR_NULL_POINTER;
  if (s.mx() && (!actq || !acts || !xq || !xs)) return MXFP4_MOE_ERR_NULL_POINTER;
  st = check_device();
  if (st) return st;
  if (!aligned(out32, 16)) return MXFP4_MOE_ERR_MISALIGNED;
  st = run_forward(s, L, x, router_logits, w13, w13s, w2, w2s, clamp_limit, out, workspace, stream, out32);
  if (st) return st;
  return copy_intermediates(s, L, workspace, act, actq, acts, xq, xs, stream);
}

int mxfp4_moe_route(const mxfp4_moe_dims* d, const float* router_logits, int32_t top_k, int32_t* ids,
                    float* weights, int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  int st = check_dims(d, top_k, true, &s);
  if (st) return st;
  if (!router_logits || !ids || !weights || !counts || !offsets || !sorted || !inv || !workspace)
    return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(router_logits, 4) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(counts, 4) ||
      !aligned(offsets, 4) || !aligned(sorted, 4) || !aligned(inv, 4) || !aligned(workspace, 256))
    return MXFP4_MOE_ERR_MISALIGNED;
  Layout L = layout_of(s);
  if (workspace_bytes < L.total) return MXFP4_MOE_ERR_WORKSPACE_TOO_SMALL;
  st = check_device();
  if (st) return st;
  if (s.T == 0) return MXFP4_MOE_OK;
  const GemmPlan plan = choose_plan(s);
  RouteArgs r = route_args(s, router_logits, workspace, L, 16 * plan.ms, 16 * plan.down_ms());
  r.ids = ids;
  r.w = weights;
  r.counts = counts;
  r.offsets = offsets;
  r.sorted = sorted;
  r.inv = inv;
  hipError_t e = launch_route(r, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MXFP4_MOE_OK;
}

static int quantize_rows(const void* in, int32_t in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                         uint8_t* scales, int fp8, hipStream_t stream) {
  if (in_dtype != MXFP4_MOE_DTYPE_BF16 && in_dtype != MXFP4_MOE_DTYPE_F32) return MXFP4_MOE_ERR_BAD_ARGUMENT;
  if (rows < 0 || K < 0) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  if (K == 0) return MXFP4_MOE_ERR_EMPTY_SHAPE;
  if (K % 32) return MXFP4_MOE_ERR_UNSUPPORTED_SHAPE;
  int64_t n;
  if (!mul_ok(rows, K, &n) || !mul_ok(n, 4, &n)) return MXFP4_MOE_ERR_SHAPE_OVERFLOW;
  if (!in || !codes || !scales) return MXFP4_MOE_ERR_NULL_POINTER;
  if (!aligned(in, 16) || !aligned(codes, 16)) return MXFP4_MOE_ERR_MISALIGNED;
  int st = check_device();
  if (st) return st;
  if (rows == 0) return MXFP4_MOE_OK;
  QuantArgs q;
  q.in = in;
  q.in_dtype = in_dtype;
  q.rows = rows;
  q.K = K;
  q.in_row_stride = K;
  q.codes = codes;
  q.scales = scales;
  q.fp8 = fp8;
  hipError_t e = launch_quantize(q, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MXFP4_MOE_OK;
}

int mxfp4_moe_quantize(const void* in, int32_t in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales, hipStream_t stream) {
  return quantize_rows(in, in_dtype, rows, K, codes, scales, 0, stream);
}

int mxfp4_moe_quantize8(const void* in, int32_t in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  return quantize_rows(in, in_dtype, rows, K, codes, scales, 1, stream);
}

}  // extern "C"
