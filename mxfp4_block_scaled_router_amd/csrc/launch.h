// Kernel argument blocks and launchers of the MXFP4 MoE layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

namespace mxmoe {

// Tuning overrides (MXFP4_MOE_PLAN, MXFP4_MOE_DECODE_VARIANT, ...) exist only in
// a library built with -DMXFP4_MOE_TUNING, for parameter sweeps; the regular
// build reads no environment and always uses the measured defaults.
inline const char* tuning_env(const char* name) {
#ifdef MXFP4_MOE_TUNING
  return getenv(name);
#else
  (void)name;
  return nullptr;
#endif
}

constexpr size_t kRouteFusedMaxLds = 48 * 1024;
// the decode gate_up kernel routes tokens itself only for E_global <= 16 x this
constexpr int kFusedRouteMaxVpl = 8;

struct RouteArgs {
  const float* logits;  // [T][E_global]
  int64_t T;
  // E_local: experts in the tables; top_k: slots per token.  With the shared
  // expert they exceed the routed local experts E_route and the router's picks
  // by one: slot t*top_k + picks of every token is on table expert E_route,
  // weight 1, id E_global.
  int32_t E_global, E_local, first_local, top_k;
  int32_t E_route, picks;
  int32_t mt1, mt2;     // token-tile heights of the gate_up and down kernels
  int32_t* ids;         // [S]
  float* w;             // [S]
  int32_t* lexp;        // [S]  local expert of each slot or -1
  int32_t* rank;        // [S]  rank within its 64-slot chunk
  int32_t* chunk_cnt;   // [ceil(S/64)][E_local]
  int32_t* counts;      // [E_local]
  int32_t* offsets;     // [E_local + 1]
  int32_t* tile_off1;   // [E_local + 1]  prefix of ceil(count / mt1)
  int32_t* tile_off2;   // [E_local + 1]  prefix of ceil(count / mt2)
  int4* tiles1;         // [tile bound 1]  {expert, rows, first sorted position, 0}
  int4* tiles2;         // [tile bound 2]
  int32_t* sorted;      // [S]
  int32_t* inv;         // [S]
  // per sorted position: token and router weight (what the down epilogue needs)
  int32_t* pos_tok;     // [S]
  float* pos_w;         // [S]
  // per tile of height mt1 (== mt2 when set): the token of each of its rows
  int32_t* tile_tok;    // [tile bound][mt1] (K-split tiles of 16 or 32 rows), or null
  // experts kept in bf16: xmap[e] >= 0 for such an expert (null: none).  They
  // keep their counts, offsets and sorted positions but get no tiles, so the
  // MXFP4 GEMMs never see them; the bf16 expert kernels cover their rows.
  const int32_t* xmap;  // [E_local]
};

struct GemmArgs {
  // activations: bf16 rows (x for gate_up, act for down) or MXFP4 rows (A4)
  const uint16_t* a_bf16;   // gate_up: x [T][H]; down: act [S][I]
  const uint8_t* a_codes;   // A4: [rows][K/2]
  const uint8_t* a_scales;  // A4: [rows][K/32]
  int64_t a_rows;           // rows of the activation tensor (T for x, S for act)
  // preshuffled weights of all local experts
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  // routing tables
  const int32_t* sorted;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tile_off;  // [E_local + 1]; tile_off[E_local] = number of tiles
  const int4* tiles;        // {expert, rows, first sorted position, 0} per tile
  const float* route_w;     // [S] (down: combine weights)
  const int32_t* pos_tok;   // [S] token of sorted position p
  const float* pos_w;       // [S] router weight of sorted position p
  const int32_t* tile_tok;  // [tile bound][16 tile_ms] token of each row of a K-split tile
  int32_t top_k, E_local;
  int64_t K, N;             // contraction length and weight rows (gate_up: N = 2I)
  float clamp_limit;
  // outputs
  uint16_t* act;            // gate_up: bf16 [S][I]
  float* out32;             // down (atomic combine): fp32 [T][H]
  float* ybuf;              // down (ordered combine): fp32 [S][H]
  // side duty: zero this fp32 buffer (grid-stride), may be null
  float* zero_buf;
  int64_t zero_n;
  // 16-row kernels: shares weighted by dispatch slot (set by the launcher)
  int32_t slot_cus;
  float slot_c;
  // K-split kernels: 16-row blocks per tile (1: 16-row tiles, 2: 32-row tiles)
  int32_t tile_ms;
  // K-split kernels: 1 = weight loads without the non-temporal hint (an
  // expert may span several tiles, whose units then find its slices in L2)
  int32_t wcache;
  // 16-row kernels with the routing inside gate_up: per down workgroup b,
  // desc[2b] = {first unit, end unit, expert, rows} and desc[2b+1] = {first
  // sorted position, tile, 0, 0} of its share, written by gate_up's first
  // workgroup from the routing it holds and read by down in place of the tile
  // count and first tile entry (two dependent loads).  Null: not used.
  int4* dn_desc;
  int32_t dn_grid, dn_fb, dn_cus;  // gate_up side: down's grid, units per tile, slot CUs
  float dn_c;                      // and slot weight
};

// Experts kept in bf16 (per-expert exclusions): weights [n][N][K] bf16, the
// j-th excluded expert in slot j.
struct XArgs {
  const uint16_t* a;        // gate_up: x [T][H]; down: act [S][I] (sorted order)
  const uint16_t* w;        // [n][N][K]
  const int32_t* xmap;      // [E_local + n]; entry E_local + j = expert of slot j
  int32_t E_local, n;
  const int32_t* counts;    // [E_local] rows per expert
  const int32_t* offsets;   // [E_local + 1] first sorted position per expert
  const int32_t* pos_tok;   // [S] token of sorted position p
  const float* pos_w;       // [S] router weight of sorted position p
  int64_t K, N;             // gate_up: K = H, N = 2I; down: K = I, N = H
  int64_t T;                // tokens: bound on the rows of one expert
  int64_t rows_per_expert;  // expected rows of one expert, T k / E_global
  float clamp_limit;
  uint16_t* act;            // gate_up: bf16 [S][I]
  float* out32;             // down, atomic combine: fp32 [T][H]
  float* ybuf;              // down, ordered combine: fp32 [S][H]
};

struct CombineArgs {
  const float* ybuf;     // [S][H]
  const float* out32;    // [T][H] (cast only)
  const float* route_w;  // [S]
  const int32_t* inv;    // [S]
  int64_t T, H;
  int32_t top_k;
  uint16_t* out;         // bf16 [T][H]
  float* out32_copy;     // ordered combine: also store the fp32 sum here (may be null)
};

struct QuantArgs {
  const void* in;
  int32_t in_dtype;      // 0 bf16, 1 f32
  int64_t rows, K;
  int64_t in_row_stride; // elements
  uint8_t* codes;        // [rows][K/2] (MXFP4) or [rows][K] (MXFP8)
  uint8_t* scales;       // [rows][K/32]
  int32_t fp8;           // 1: E4M3 elements (MXFP8)
};

// fp32 / bf16 weights [E][N][K] -> preshuffled MXFP4 in one pass
struct QuantPreshuffleArgs {
  const void* in;
  int32_t in_dtype;              // 0 bf16, 1 f32
  uint8_t* codes;
  uint8_t* scales;
  int64_t E, N, K;
  int32_t interleave_gate_up;    // 1 for w13
};

struct PreshuffleArgs {
  const uint8_t* canon_codes;   // [E][N][K/2]
  const uint8_t* canon_scales;  // [E][N][K/32]
  uint8_t* codes;
  uint8_t* scales;
  int64_t E, N, K;
  int32_t interleave_gate_up;   // 1 for w13
};

// variant of the grouped GEMMs chosen by the host
struct GemmPlan {
  int ksplit = 0; // 1: the K-split kernels (decode.hip), tiles of 16 ms rows, ms 1 or 2
  int ms;        // 16-row token subtiles per workgroup (token tile = 16 * ms)
  int fg;        // 16-feature groups per wave
  int nw;        // waves per workgroup
  int ms_dn = 0; // down's token tile in 16-row subtiles when it differs from gate_up's (0: ms)
  int dw = 0;    // 320-row tiles: gate_up on the direct-weight tiles
  int dw_dn = 0; // 320-row tiles: down on the direct-weight tiles
  int down_ms() const { return ms_dn ? ms_dn : ms; }
};

hipError_t launch_route(const RouteArgs& a, hipStream_t stream);
// whether the routing of a is small enough for the decode gate_up kernel to
// route the tokens itself in each workgroup
bool route_fusable(const RouteArgs& a);
hipError_t launch_gate_up(const GemmArgs& a, const GemmPlan& p, int64_t max_tiles, bool a4,
                          hipStream_t stream);
hipError_t launch_down(const GemmArgs& a, const GemmPlan& p, int64_t max_tiles, bool a4,
                       bool ordered, hipStream_t stream);
// route non-null: every workgroup routes the tokens itself first (no routing
// kernel before it); only when route_fusable(*route)
// af: activation format, 0 bf16, 1 MXFP4 (A4), 2 MXFP8 (A8)
hipError_t launch_gate_up_ksplit(const GemmArgs& a, const RouteArgs* route, int64_t max_tiles, int af,
                                 hipStream_t stream);
// Large token tiles through an LDS ring fed by global->LDS copies (tile.hip):
// mt = 128 (128 x 512 tiles) or, with MX activations, 320 (320 x 128 tiles);
// dw: with MXFP4 activations and mt = 320, the direct-weight 320 x 256 tiles
// (weights loaded into registers, activations through LDS)
hipError_t launch_gate_up_tile(const GemmArgs& a, int64_t max_tiles, int af, int mt, bool dw,
                               hipStream_t stream);
hipError_t launch_down_tile(const GemmArgs& a, int64_t max_tiles, int af, int mt, bool dw, bool ordered,
                            hipStream_t stream);
// whether the tile kernels of height mt (dw: the direct-weight tiles) take a
// contraction of length K with activation format af (the 320-row tiles hold
// their rows' scale bytes in LDS)
bool tile_fits(int af, int mt, int64_t K, bool dw = false);
// The grid and share parameters launch_down_ksplit will use for these
// arguments (for the gate_up side of dn_desc).
hipError_t down_ksplit_shares(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, int* grid, int* fb,
                              int* cus, float* c);
// whether the K-split kernels hold the activations of two 16-row blocks
// (32-row tiles) in registers for contraction length K and activation format af
bool ksplit_two_blocks_fit(int64_t K, int af);
hipError_t launch_down_ksplit(const GemmArgs& a, int64_t max_tiles, int af, bool ordered,
                              hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, bool ordered, hipStream_t stream);
// The expert map of the excluded experts from a bit set of E experts passed by
// value: map[e] = bf16 slot of expert e (its rank among the excluded) or -1,
// map[E + j] = expert of slot j.
constexpr int kExpertMapMax = 544;  // 17 words
struct ExpertMapArgs {
  uint32_t bits[kExpertMapMax / 32];
  int32_t E;
};
hipError_t launch_expert_map(const ExpertMapArgs& m, int32_t* map, hipStream_t stream);
// gate_up + SwiGLU and down + combine of the experts kept in bf16 (bf16x.hip)
hipError_t launch_bf16x_gate_up(const XArgs& a, hipStream_t stream);
hipError_t launch_bf16x_down(const XArgs& a, bool ordered, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_preshuffle(const PreshuffleArgs& a, hipStream_t stream);
hipError_t launch_quantize_preshuffle(const QuantPreshuffleArgs& a, hipStream_t stream);
hipError_t launch_copy_rows(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);

}  // namespace mxmoe
